"""Pins of the oracle's YaRN RoPE (page "DeepSeek-V2 paper summary", section 3.1.4: s = 40,
alpha = 1, beta = 32, sqrt(t) = 0.0707 ln s + 1; the frequency ramp is the YaRN paper's, which the
page cites).  Each pin is a property that any correct reading must have and that is checked
through plain RoPE angles or closed forms, not through the ramp formula itself:
  * s = 1 is plain RoPE;
  * pairs that turn more than beta times over the original context rotate exactly as before;
  * pairs that turn fewer than alpha times are position-interpolated: the angle at position m*s
    is the plain angle at m;
  * in between, the frequency lies strictly between theta/s and theta, and the interpolated
    share is an affine function of the number of turns;
  * at DeepSeek-V2 sizes the three regimes hold 11, 12 and 9 pairs (closed form below);
  * the logit factor is 1 without YaRN and (0.0707 ln 40 + 1)^2 at s = 40;
  * it is still a rotation (norms kept) and scores still depend only on relative position.
Planted mistakes in a copy of the oracle must fail them."""
import dataclasses
import inspect
import math
import types

import numpy as np
import pytest

import mla_synth as S
import oracle.mla_oracle as O

V2Y = S.V2_YARN


def _plain(pos, d_hr=64, base=10000.0):
    return O.rope_angles(pos, d_hr, base)


def _turns(d_hr=64, base=10000.0, L=4096):
    """Number of full turns each pair makes over L positions (plain frequencies)."""
    return _plain(L, d_hr, base) / (2 * math.pi)


def _regime_pins(mod):
    yarn = mod.yarn_of(V2Y)
    assert yarn == (40.0, 4096, 1.0, 32.0)
    turns = _turns()
    fast, slow = turns > 32.0, turns < 1.0
    mid = ~fast & ~slow
    # closed form: turns_k = 4096 / (2 pi) * 10000^(-k/32) > 32 <=> k < 32 ln(4096 / (64 pi)) / ln 10000
    k_fast = 32 * math.log(4096 / (64 * math.pi)) / math.log(10000)
    k_slow = 32 * math.log(4096 / (2 * math.pi)) / math.log(10000)
    assert int(fast.sum()) == math.ceil(k_fast) == 11
    assert int(slow.sum()) == 32 - math.ceil(k_slow) == 9
    assert int(mid.sum()) == 12
    m = np.arange(0, 200000, 977, dtype=np.int64)
    ya = mod.rope_angles(m, 64, 10000.0, yarn)
    pa = _plain(m)
    assert np.array_equal(ya[:, fast], pa[:, fast])
    # interpolated pairs: the angle at position m * s is the plain angle at m
    np.testing.assert_allclose(mod.rope_angles(m * 40, 64, 10000.0, yarn)[:, slow], pa[:, slow], rtol=1e-13)
    ratio = (mod.rope_angles(1, 64, 10000.0, yarn) / _plain(1))
    assert np.all(ratio[mid] > 1 / 40) and np.all(ratio[mid] < 1.0)
    # interpolated share g = (ratio - 1/s) / (1 - 1/s) is affine in the number of turns
    g = (ratio[mid] - 1 / 40) / (1 - 1 / 40)
    slope = np.diff(g) / np.diff(turns[mid])
    np.testing.assert_allclose(slope, slope[0], rtol=1e-9)
    assert slope[0] > 0


def _plain_when_off(mod):
    assert mod.yarn_of(S.V2) is None
    m = np.arange(0, 5000, 7)
    assert np.array_equal(mod.rope_angles(m, 64, 10000.0, mod.yarn_of(S.V2)), _plain(m))
    theta = _plain(1)
    np.testing.assert_allclose(mod.yarn_frequencies(theta, 1.0, 4096, 1.0, 32.0), theta, rtol=1e-15)


def _logit_factor(mod):
    assert mod.yarn_logit_factor(S.V2) == 1.0
    t = (0.0707 * math.log(40.0) + 1.0) ** 2
    assert abs(mod.yarn_logit_factor(V2Y) - t) < 1e-12
    assert abs(t - 1.5897) < 1e-4
    assert abs(mod.softmax_scale(V2Y) - t / math.sqrt(192.0)) < 1e-12
    fixed = dataclasses.replace(V2Y, softmax_scale=0.125)
    assert mod.softmax_scale(fixed) == 0.125  # a layer-fixed scale is taken as given


def test_plain_rope_when_yarn_is_off():
    _plain_when_off(O)


def test_regimes_interpolation_and_ramp():
    _regime_pins(O)


def test_logit_factor():
    _logit_factor(O)


def test_still_a_rotation_with_relative_positions():
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    y = O.yarn_of(V2Y)
    rq = O.apply_rope(np.stack([q] * 3), np.array([5, 7000, 150000]), 10000.0, y)
    assert np.allclose(np.linalg.norm(rq, axis=1), np.linalg.norm(q))
    d1 = O.apply_rope(q, 9000, 10000.0, y) @ O.apply_rope(k, 8000, 10000.0, y)
    d2 = O.apply_rope(q, 121000, 10000.0, y) @ O.apply_rope(k, 120000, 10000.0, y)
    assert abs(d1 - d2) < 1e-9 * (np.abs(q) @ np.abs(k))


def test_query_and_key_use_the_same_frequencies():
    dims = S.TINY_YARN
    W = S.make_weights(dims)
    h = S.hidden_history(dims, 0, 40, "normal002").astype(np.float64)
    pos = np.arange(40)
    kr = O.latent_entries(W, dims, h, pos)[:, dims.d_c:]
    want = O.apply_rope(h @ np.asarray(W["W_KR"], np.float64).T, pos, dims.rope_base, O.yarn_of(dims))
    assert np.array_equal(kr, want)
    qc, qr = O.query(W, dims, h, pos)
    plain = O.query(W, dataclasses.replace(dims, rope_scale=1.0), h, pos)[1]
    assert np.array_equal(qc, O.query(W, dataclasses.replace(dims, rope_scale=1.0), h, pos)[0])
    assert not np.allclose(qr, plain)


MUTATIONS = {
    "ramp_reversed": ("gamma = np.clip((rotations - alpha) / (beta - alpha), 0.0, 1.0)",
                      "gamma = 1.0 - np.clip((rotations - alpha) / (beta - alpha), 0.0, 1.0)"),
    "stretched_not_interpolated": ("return (1.0 - gamma) * theta / s + gamma * theta",
                                   "return (1.0 - gamma) * theta * s + gamma * theta"),
    "turns_from_frequency": ("rotations = np.float64(orig_ctx) / wavelength",
                             "rotations = np.float64(orig_ctx) / theta"),
    "factor_not_squared": ("return float(root_t * root_t)", "return float(root_t)"),
    "ramp_on_wavelength": ("gamma = np.clip((rotations - alpha) / (beta - alpha), 0.0, 1.0)",
                           "gamma = np.clip((wavelength - alpha) / (beta - alpha), 0.0, 1.0)"),
}


def _mutant(name):
    src = inspect.getsource(O)
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType("yarn_mutant_" + name)
    exec(compile(src.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(name)
    with np.errstate(all="ignore"), pytest.raises(AssertionError):
        _plain_when_off(mod)
        _regime_pins(mod)
        _logit_factor(mod)
