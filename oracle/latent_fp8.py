"""fp8 latent cache for the oracle: per-token-scaled e4m3 codes of the cached entries.

TEST INFRASTRUCTURE ONLY (see mla_oracle.py): only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module, and it shares no code with the HIP path.

What it follows: the page "DeepSeek-V2 paper summary", section 3.2.3, serves V2 with the KV cache
quantised to about 6 bits per element on average (citing KVQuant); the pages give no format.
The plainest reading that an MI355X path can serve natively (the design notes list it):
  * each cached entry [c_KV | k_R] (App. C) is first formed as in the bf16 path (rounded to
    bf16), then each of its two parts gets one fp32 scale per token, s = amax(|part|) / 448
    (448 = the largest finite e4m3 value), and every element x of the part is stored as the e4m3
    code of x / s (fp32 division), rounded to nearest, ties to even, saturating at +-448; a part
    that is all zero gets s = 0 and zero codes;
  * e4m3 is the OCP 8-bit float "E4M3": sign, 4 exponent bits with bias 7, 3 mantissa bits,
    subnormals at exponent 0 (m * 2^-9), no infinities, the all-ones exponent and mantissa is NaN;
  * attention reads value(code) * s; the quantiser's decisions are integers and are taken in
    fp32, the precision the kernels use.
Pins: the code table and the encoder against torch's float8_e4m3fn conversion (a library
routine), the error bound of the format, and the amax element mapping to +-448.  The decode step
(mla_decode_fp8) is pinned against the plain decode step of mla_oracle on entries that quantise
exactly, and its new codes against the quantised prefill row of the same token.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_value(code) -> np.ndarray:
    """Value of e4m3 codes (uint8 array) in fp64, NaN for the two NaN codes."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.power(2.0, e - 7.0))
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


_POS_CODES = np.arange(0x7F, dtype=np.uint8)      # 0x00 .. 0x7E: the non-negative finite codes
_POS_VALUES = e4m3_value(_POS_CODES)               # increasing with the code


def e4m3_encode(x) -> np.ndarray:
    """e4m3 codes of x (taken as fp32): nearest value, ties to the even code, saturating at
    +-448; NaN -> 0x7F.  Zero and values below half the smallest subnormal encode as +-0."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def quantize_part(x) -> tuple:
    """One part of an entry (its values as fp32): (codes, s) with s = amax / 448 in fp32 and
    codes = e4m3(x / s) with the division in fp32."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    if amax == 0:
        return np.zeros(x.shape, np.uint8), np.float32(0)
    s = np.float32(amax / np.float32(E4M3_MAX))
    return e4m3_encode((x / s).astype(np.float32)), s


def quantize_entries(entries, d_c: int) -> tuple:
    """Entries [n, d_c + d_hr] (values representable in fp32, e.g. bf16-rounded) ->
    codes [n, d_c + d_hr] uint8 and scales [n, 2] fp32 = (s_c, s_r) per token."""
    entries = np.asarray(entries, dtype=np.float32)
    n = entries.shape[0]
    codes = np.zeros(entries.shape, np.uint8)
    scales = np.zeros((n, 2), np.float32)
    for t in range(n):
        codes[t, :d_c], scales[t, 0] = quantize_part(entries[t, :d_c])
        codes[t, d_c:], scales[t, 1] = quantize_part(entries[t, d_c:])
    return codes, scales


def dequantize(codes, scales, d_c: int) -> np.ndarray:
    """Values attention reads: value(code) * s of the part, in fp64."""
    v = e4m3_value(codes)
    scales = np.asarray(scales, dtype=np.float64)
    v[..., :d_c] *= scales[..., 0:1]
    v[..., d_c:] *= scales[..., 1:2]
    return v


def bf16_round(x) -> np.ndarray:
    """Round to the nearest bf16 (ties to even), returned as fp32: the entry as the bf16 path
    stores it, which the quantiser then takes as input."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def mla_decode_fp8(W: dict, dims, h_new, cache_codes, cache_scales) -> dict:
    """One decode step over fp8 caches (un-absorbed form of App. C, like mla_oracle.mla_decode):
    the new token's entry is formed, rounded to bf16 and quantised; every head then attends
    over the dequantised entries of the L_b + 1 tokens.
    cache_codes[b] [L_b, d_c + d_hr] uint8, cache_scales[b] [L_b, 2].
    Returns u, o, lse as mla_decode does, plus the new entry's codes [B, entry] and scales [B, 2]."""
    from oracle import mla_oracle as O
    h_new = np.asarray(h_new, dtype=np.float64)
    B = h_new.shape[0]
    u = np.zeros((B, dims.d_model))
    o = np.zeros((B, dims.n_h, dims.d_h))
    lse = np.zeros((B, dims.n_h))
    codes_new = np.zeros((B, dims.entry), np.uint8)
    scales_new = np.zeros((B, 2), np.float32)
    for b in range(B):
        L = int(np.asarray(cache_codes[b]).shape[0])
        e = O.latent_entries(W, dims, h_new[b:b + 1], np.array([L]))
        c, s = quantize_entries(bf16_round(e), dims.d_c)
        codes_new[b], scales_new[b] = c[0], s[0]
        codes = np.concatenate([np.asarray(cache_codes[b], np.uint8).reshape(L, dims.entry), c])
        scales = np.concatenate([np.asarray(cache_scales[b], np.float32).reshape(L, 2), s])
        full = dequantize(codes, scales, dims.d_c)
        qc, qr = O.query(W, dims, h_new[b:b + 1], np.array([L]))
        ob, lb = O.attend_unabsorbed(W, dims, qc, qr, full, np.array([L + 1]))
        o[b], lse[b] = ob[0], lb[0]
        u[b] = O.output(W, dims, ob)[0]
    return {"u": u, "o": o, "lse": lse, "codes": codes_new, "scales": scales_new}
