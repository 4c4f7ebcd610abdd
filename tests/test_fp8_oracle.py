"""Pins of the fp8 latent-cache oracle (oracle/latent_fp8.py) against things it does not share
code with: torch's float8_e4m3fn conversion (a library routine) for the code table and the
encoder, the error bound of a 3-mantissa-bit format, the amax element landing on +-448, and
planted mistakes that these pins must reject."""
import inspect
import types

import numpy as np
import pytest
import torch

import oracle.latent_fp8 as F


def _torch_encode(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_value(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def _table_pins(mod):
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = mod.e4m3_value(codes), _torch_value(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.nanmax(ours) == 448.0 and np.nanmin(np.abs(ours[ours != 0])) == 2.0 ** -9


def _encode_pins(mod):
    rng = np.random.default_rng(11)
    # log-uniform magnitudes across the subnormal and normal ranges, both signs
    mag = np.exp2(rng.uniform(-13.0, np.log2(448.0), 20000))
    x = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    # every representable value, and every midpoint between neighbours (the ties)
    vals = mod.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, vals.astype(np.float32), mids, -mids, np.float32([0.0, -0.0, 448.0, -448.0])])
    assert np.array_equal(mod.e4m3_encode(x), _torch_encode(x))


def test_code_table_matches_torch():
    _table_pins(F)


def test_encoder_matches_torch_including_ties():
    _encode_pins(F)


def test_encoder_saturates():
    x = np.float32([449.0, 480.0, 1e6, -1e6, 447.9])
    assert list(F.e4m3_encode(x)) == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E]


def test_quantized_part_error_bound_and_amax():
    rng = np.random.default_rng(5)
    for scale in (1e-3, 1.0, 37.0):
        x = (rng.standard_normal(512) * scale).astype(np.float32)
        codes, s = F.quantize_part(x)
        deq = F.e4m3_value(codes) * np.float64(s)
        # half an ulp of a 3-bit mantissa (relative 2^-4) in the normal range, 2^-10 s below it
        err = np.abs(deq - x.astype(np.float64))
        assert np.all(err <= 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * s * (1 + 1e-6))
        i = int(np.argmax(np.abs(x)))
        assert codes[i] & 0x7F == 0x7E
        assert abs(deq[i] - x[i]) <= 1e-6 * abs(x[i])


def test_zero_part_and_entry_layout():
    e = np.zeros((2, 576), np.float32)
    e[1, 512:] = np.linspace(-1, 1, 64)
    codes, scales = F.quantize_entries(e, 512)
    assert scales[0, 0] == 0 and scales[0, 1] == 0 and not codes[0].any()
    assert scales[1, 0] == 0 and scales[1, 1] == np.float32(np.float32(1.0) / np.float32(448.0))
    back = F.dequantize(codes, scales, 512)
    assert np.allclose(back[1, 512:], e[1, 512:], atol=2.0 ** -4)


def test_bf16_round_matches_torch():
    x = np.random.default_rng(3).standard_normal(10000).astype(np.float32) * 7
    assert np.array_equal(F.bf16_round(x), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


MUTATIONS = {
    "exponent_bias": ("np.power(2.0, e - 7.0)", "np.power(2.0, e - 8.0)"),
    "subnormal_scale": ("m * 2.0 ** -9", "m * 2.0 ** -10"),
    "ties_away_from_zero": ("(dhi == dlo) & (_POS_CODES[hi] % 2 == 0)", "(dhi == dlo)"),
    "truncation": ("pick_hi = (dhi < dlo) |", "pick_hi = (dhi == 0) & (dhi < dlo) |"),
    "lost_sign": ("code = np.where(np.signbit(x), code | 0x80, code)", "code = code"),
}


def _mutant(name):
    src = inspect.getsource(F)
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType("fp8_mutant_" + name)
    exec(compile(src.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(name)
    with pytest.raises(AssertionError):
        _table_pins(mod)
        _encode_pins(mod)
