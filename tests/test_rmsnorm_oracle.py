"""Pins of the oracle's latent RMSNorm (page "DeepSeek-V2 paper summary", section 3.1.2: RMSNorm
layers after the compressed latent vectors).  Checked against torch's rms_norm in fp64 (a library
routine), against its closed forms (unit mean square with unit gain, invariance to the input's
scale, the gain acting elementwise, a zero row staying zero), and for where it acts in the layer:
on c^q before both query products and on c^KV before caching, never on the rope key.  Planted
mistakes in a copy of the oracle must fail them."""
import dataclasses
import inspect
import types

import numpy as np
import pytest
import torch

import mla_synth as S
import oracle.mla_oracle as O


def _library(x, g, eps):
    t = torch.from_numpy(np.asarray(x, np.float64))
    return torch.nn.functional.rms_norm(t, (t.shape[-1],), torch.from_numpy(np.asarray(g, np.float64)),
                                        eps).numpy()


def _norm_pins(mod):
    rng = np.random.default_rng(2)
    for W, eps in ((512, 1e-6), (1536, 1e-6), (32, 1e-3)):
        x = rng.standard_normal((7, W)) * np.geomspace(1e-3, 1e2, 7)[:, None]
        g = 1 + 0.1 * rng.standard_normal(W)
        np.testing.assert_allclose(mod.rms_norm(x, g, eps), _library(x, g, eps), rtol=1e-12, atol=1e-15)
        y = mod.rms_norm(x, np.ones(W), 0.0)
        np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-12)
        np.testing.assert_allclose(mod.rms_norm(37.5 * x, g, 0.0), mod.rms_norm(x, g, 0.0), rtol=1e-12)
        np.testing.assert_allclose(mod.rms_norm(x, g, eps), mod.rms_norm(x, np.ones(W), eps) * g, rtol=1e-13)
    z = mod.rms_norm(np.zeros((2, 16)), np.ones(16), 1e-6)
    assert np.all(z == 0.0)


def _placement_pins(mod):
    dims = S.TINY_NORM
    W = S.make_weights(dims)
    assert "g_cq" in W and "g_ckv" in W
    h = S.hidden_history(dims, 0, 12, "normal002").astype(np.float64)
    pos = np.arange(12)
    plainW = {k: v for k, v in W.items() if not k.startswith("g_")}
    ent, ent0 = mod.latent_entries(W, dims, h, pos), mod.latent_entries(plainW, dims, h, pos)
    assert np.array_equal(ent[:, dims.d_c:], ent0[:, dims.d_c:])  # the rope key is not normalised
    np.testing.assert_allclose(ent[:, :dims.d_c], _library(ent0[:, :dims.d_c], W["g_ckv"], dims.rms_eps),
                               rtol=1e-12)
    # both query products read the normalised c^q: compare with the plain layer fed the
    # normalised c^q through weights that absorb W_DQ (W_DQ := I on a d_cq-wide input)
    cq = _library(h @ np.asarray(W["W_DQ"], np.float64).T, W["g_cq"], dims.rms_eps)
    qc, qr = mod.query(W, dims, h, pos)
    eye = dict(plainW, W_DQ=np.eye(dims.d_cq))
    dims_eye = dataclasses.replace(dims, d_model=dims.d_cq)
    qc2, qr2 = mod.query(eye, dims_eye, cq, pos)
    np.testing.assert_allclose(qc, qc2, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(qr, qr2, rtol=1e-12, atol=1e-15)


def test_rms_norm_matches_library_and_closed_forms():
    _norm_pins(O)


def test_norm_placement_in_the_layer():
    _placement_pins(O)


def test_no_query_norm_without_query_compression():
    dims = S.V2_LITE_NORM
    W = S.make_weights(dims)
    assert "g_cq" not in W and "g_ckv" in W


MUTATIONS = {
    "sum_not_mean": ("ms = np.mean(x * x, axis=-1, keepdims=True)", "ms = np.sum(x * x, axis=-1, keepdims=True)"),
    "eps_outside_root": ("return x / np.sqrt(ms + eps) * np.asarray(gain, dtype=np.float64)",
                         "return x / (np.sqrt(ms) + eps) * np.asarray(gain, dtype=np.float64)"),
    "gain_divides": ("return x / np.sqrt(ms + eps) * np.asarray(gain, dtype=np.float64)",
                     "return x / np.sqrt(ms + eps) / np.asarray(gain, dtype=np.float64)"),
    "norm_over_rows": ("ms = np.mean(x * x, axis=-1, keepdims=True)", "ms = np.mean(x * x, axis=0, keepdims=True)"),
    "norm_on_the_whole_entry": (
        "    return np.concatenate([ckv, kr], axis=1)",
        "    e = np.concatenate([ckv, kr], axis=1)\n"
        "    return rms_norm(e, np.ones(e.shape[1]), dims.rms_eps) if \"g_ckv\" in W else e"),
    "query_norm_dropped": ("        cq = rms_norm(cq, _w(W, \"g_cq\"), dims.rms_eps)", "        pass"),
}


def _mutant(name):
    src = inspect.getsource(O)
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType("norm_mutant_" + name)
    exec(compile(src.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(name)
    with np.errstate(all="ignore"), pytest.raises(AssertionError):
        _norm_pins(mod)
        _placement_pins(mod)
