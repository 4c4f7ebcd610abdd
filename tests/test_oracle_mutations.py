"""Plants plausible mistakes in a copy of the oracle (on the CPU) and checks that the
pins in test_oracle.py reject every one of them: a wrong sign, a dropped term, a
transposed or swapped operand, a wrong head split, an off-by-one causal bound, a wrong
RoPE frequency or position, a wrong logit scale and a softmax without max subtraction."""
import inspect
import types

import numpy as np
import pytest

import mla_synth as S
import oracle.mla_oracle as O
from tests import test_oracle as T

MUTATIONS = {
    "rope_sign": ("out[..., 0::2] = xe * c - xo * s", "out[..., 0::2] = xe * c + xo * s"),
    "rope_freq": ("-2.0 * k / d_hr", "-1.0 * k / d_hr"),
    "dropped_rope_score": ("qc[:, i, :] @ Kc.T + qr[:, i, :] @ kr.T", "qc[:, i, :] @ Kc.T"),
    "swapped_up_projection": ("Kc = c @ WUK[rows].T", "Kc = c @ WUV[rows].T"),
    "transposed_head_split": (
        "qc = (cq @ _w(W, \"W_UQ\").T).reshape(h.shape[0], dims.n_h, dims.d_h)",
        "qc = (cq @ _w(W, \"W_UQ\").T).reshape(h.shape[0], dims.d_h, dims.n_h).transpose(0, 2, 1)"),
    "causal_off_by_one": ("o, lse = attend(W, dims, qc, qr, cache, idx + 1)",
                          "o, lse = attend(W, dims, qc, qr, cache, np.maximum(idx, 1))"),
    "rope_on_wrong_position": ("kr = apply_rope(h @ _w(W, \"W_KR\").T, np.asarray(pos), dims.rope_base, yarn_of(dims))",
                               "kr = apply_rope(h @ _w(W, \"W_KR\").T, np.asarray(pos) + 1, dims.rope_base, yarn_of(dims))"),
    "wrong_scale": ("return 1.0 / np.sqrt(np.float64(dims.d_h + dims.d_hr))",
                    "return 1.0 / np.sqrt(np.float64(dims.d_h))"),
    "no_max_subtraction": ("    e = np.exp(s - m)\n", "    e = np.exp(s - m * 0.0)\n    e = e * np.exp(-m)\n"),
    "value_from_rope_part": ("c, kr = cache[:, : dims.d_c], cache[:, dims.d_c:]\n    n = qc.shape[0]\n    L = cache.shape[0]\n    kv_len = np.asarray(kv_len)\n    mask = np.arange(L)[None, :] < kv_len[:, None]  # [n, L]",
                             "c, kr = cache[:, : dims.d_c], cache[:, dims.d_c:]\n    c = np.roll(c, 1, axis=1)\n    n = qc.shape[0]\n    L = cache.shape[0]\n    kv_len = np.asarray(kv_len)\n    mask = np.arange(L)[None, :] < kv_len[:, None]  # [n, L]"),
}


def _mutant(name):
    src = inspect.getsource(O)
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType("oracle_mutant_" + name)
    exec(compile(src.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    return mod


def _pins_pass(mod, monkeypatch):
    monkeypatch.setattr(T, "O", mod)
    try:
        T.test_bruteforce_scalar_layer(5)
        T.test_bruteforce_scalar_layer(0)
        T.test_reduces_to_textbook_mha()
        T.test_attention_matches_torch_sdpa_fp64()
        T.test_rope_complex_closed_form()
        T.test_softmax_rows_sum_to_one_and_overflow()
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    with np.errstate(all="ignore"):
        assert not _pins_pass(_mutant(name), monkeypatch), name


def test_unmutated_copy_passes(monkeypatch):
    mod = types.ModuleType("oracle_copy")
    exec(compile(inspect.getsource(O), mod.__name__, "exec"), mod.__dict__)
    assert _pins_pass(mod, monkeypatch)
