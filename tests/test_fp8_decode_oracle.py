"""Pins of the fp8 decode step of the oracle (oracle/latent_fp8.mla_decode_fp8), the expected
value of the fp8-cache decode tests on the GPU.  It composes four steps: form the new token's
entry at its position, round it to bf16, quantise it, and attend over the dequantised entries
of all L + 1 tokens (the low-bit cache of the serving section, 3.2.3 of the page "DeepSeek-V2
paper summary"; the reading is the one in oracle/latent_fp8.py).  Two pins, each against a
function pinned elsewhere:

  * exact entries: when the new token's entry is exactly (code x scale) for some e4m3 code and a
    power-of-two scale, quantisation loses nothing, so the fp8 step must equal the plain decode
    step (mla_oracle.mla_decode, pinned by brute force, textbook MHA and torch SDPA) run on the
    dequantised history, to rounding;
  * the new codes: the codes and scales of the new token must be those of the bf16-rounded cache
    row that the oracle's prefill (pinned the same way) forms for the same token at the same
    position.

Planted mistakes (rope at the next position, quantising before rounding, codes or scales of the
new token concatenated at the wrong end, the query at the wrong position, the token not
attending to itself) must fail one of them."""
import dataclasses
import inspect
import types

import numpy as np
import pytest

import mla_synth as S
import oracle.latent_fp8 as F
import oracle.mla_oracle as O

DIMS = S.TINY
DIMS_NOQ = dataclasses.replace(S.TINY, d_cq=0)  # no query compression (App. B.1 reading)
DIMS_YARN = S.TINY_YARN


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _exact_case(dims, lens, seed):
    """Weights whose latent columns at the new tokens' one-hot inputs are e4m3 values times 2^-8
    (amax exactly 448 * 2^-8), with a zero rope-key column there; random fp8 histories."""
    rng = np.random.default_rng(seed)
    W = {k: v.astype(np.float64) for k, v in S.make_weights(dims).items()}
    B = len(lens)
    ks = rng.choice(dims.d_model, size=B, replace=False)
    grid = F.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    for k in ks:
        col = grid[rng.integers(1, 0x7F, dims.d_c)] * rng.choice([-1.0, 1.0], dims.d_c)
        col[rng.integers(dims.d_c)] = 448.0 * rng.choice([-1.0, 1.0])
        W["W_DKV"][:, k] = col * 2.0 ** -8
        W["W_KR"][:, k] = 0.0
    h_new = np.zeros((B, dims.d_model))
    h_new[np.arange(B), ks] = 1.0
    codes = [S.fp8_codes(L, dims.entry, seed=100 + b) for b, L in enumerate(lens)]
    scales = [S.fp8_scales(L, seed=200 + b) for b, L in enumerate(lens)]
    return W, h_new, codes, scales


def _exact_entries_pin(mod, dims, lens, seed=0):
    W, h_new, codes, scales = _exact_case(dims, lens, seed)
    got = mod.mla_decode_fp8(W, dims, h_new, codes, scales)
    caches = [F.dequantize(c, s, dims.d_c) for c, s in zip(codes, scales)]
    ref = O.mla_decode(W, dims, h_new, caches)
    for key in ("u", "o", "lse"):
        assert _rel(got[key], ref[key]) <= 1e-12, key
    # nothing was lost in quantising the new entry
    back = F.dequantize(got["codes"], got["scales"], dims.d_c)
    assert np.array_equal(back, ref["entry"])


def _new_codes_pin(mod, dims, L, seed=0):
    W = {k: v.astype(np.float64) for k, v in S.make_weights(dims).items()}
    h = S.hidden_history(dims, seed, L + 1, "unit").astype(np.float64)
    full = O.mla_prefill(W, dims, h)["cache"]
    hist_codes, hist_scales = F.quantize_entries(F.bf16_round(full[:L]), dims.d_c)
    got = mod.mla_decode_fp8(W, dims, h[L:], [hist_codes], [hist_scales])
    want_codes, want_scales = F.quantize_entries(F.bf16_round(full[L:]), dims.d_c)
    assert np.array_equal(got["scales"], want_scales)
    assert np.array_equal(got["codes"], want_codes)


@pytest.mark.parametrize("dims", [DIMS, DIMS_NOQ, DIMS_YARN], ids=["tiny", "tiny_noq", "tiny_yarn"])
def test_fp8_decode_equals_plain_decode_on_exact_entries(dims):
    _exact_entries_pin(F, dims, lens=[0, 1, 7, 70])


@pytest.mark.parametrize("L", [0, 1, 15, 64, 300])
@pytest.mark.parametrize("dims", [DIMS, DIMS_YARN], ids=["tiny", "tiny_yarn"])
def test_fp8_decode_new_codes_match_prefill_row(dims, L):
    _new_codes_pin(F, dims, L)


MUTATIONS = {
    "rope_at_next_position": ("e = O.latent_entries(W, dims, h_new[b:b + 1], np.array([L]))",
                              "e = O.latent_entries(W, dims, h_new[b:b + 1], np.array([L + 1]))"),
    "quantise_before_rounding": ("quantize_entries(bf16_round(e), dims.d_c)", "quantize_entries(e, dims.d_c)"),
    "new_codes_first": ("codes = np.concatenate([np.asarray(cache_codes[b], np.uint8).reshape(L, dims.entry), c])",
                        "codes = np.concatenate([c, np.asarray(cache_codes[b], np.uint8).reshape(L, dims.entry)])"),
    "new_scales_first": ("scales = np.concatenate([np.asarray(cache_scales[b], np.float32).reshape(L, 2), s])",
                         "scales = np.concatenate([s, np.asarray(cache_scales[b], np.float32).reshape(L, 2)])"),
    "query_at_next_position": ("qc, qr = O.query(W, dims, h_new[b:b + 1], np.array([L]))",
                               "qc, qr = O.query(W, dims, h_new[b:b + 1], np.array([L + 1]))"),
    "self_not_attended": ("O.attend_unabsorbed(W, dims, qc, qr, full, np.array([L + 1]))",
                          "O.attend_unabsorbed(W, dims, qc, qr, full, np.array([max(L, 1)]))"),
}


def _mutant(name):
    src = inspect.getsource(F)
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType("fp8_decode_mutant_" + name)
    exec(compile(src.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    return mod


def _pins_pass(mod):
    try:
        for dims in (DIMS, DIMS_YARN):
            _exact_entries_pin(mod, dims, lens=[0, 1, 7, 70])
            for L in (1, 15, 64):
                _new_codes_pin(mod, dims, L)
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    with np.errstate(all="ignore"):
        assert not _pins_pass(_mutant(name)), name


def test_unmutated_copy_passes():
    mod = types.ModuleType("fp8_decode_copy")
    exec(compile(inspect.getsource(F), mod.__name__, "exec"), mod.__dict__)
    assert _pins_pass(mod)
