"""Seeded synthetic inputs for the MLA layer: dimensions, weights, hidden states,
page permutations and ragged context lengths.

This module is shared by the fp64 oracle's tests and by the GPU path's tests and
benchmark.  It holds no step of the attention method itself: it only draws
random numbers, applies the input recipe (RMS normalisation of the hidden
states, rounding to bf16) and fixes the dimension presets.

Dimensions follow the DeepSeek-V2 summary page (7shi.hateblo.jp, "DeepSeek-V2"
paper summary): section 3.1.2 (hyper-parameters: d=5120, n_h=128, d_h=128,
d_c=512, d'_q=1536, d_e=64) and App. B.1 (V2-Lite: d=2048, 16 heads x 128,
d_c=512, no query compression, d_e=64).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

F32 = "f32"
BF16 = "bf16"

# Fixed order in which the weight matrices are drawn from the weight generator.
WEIGHT_ORDER = ("W_DQ", "W_UQ", "W_QR", "W_DKV", "W_KR", "W_UK", "W_UV", "W_O")

SEED_WEIGHTS = 0
SEED_HISTORY = 1
SEED_PAGES = 2
SEED_LENGTHS = 3
SEED_STEP = 4
SEED_GAINS = 6


@dataclasses.dataclass(frozen=True)
class Dims:
    """One MLA layer's sizes.  d_cq == 0 means no query compression (c^q := h)."""

    d_model: int
    n_h: int
    d_h: int
    d_c: int
    d_cq: int
    d_hr: int
    dtype: str = BF16
    rope_base: float = 10000.0
    softmax_scale: float = 0.0  # 0: the layer's default scale
    # YaRN context extension (off unless rope_scale > 1): scale s, original context length L,
    # ramp bounds alpha, beta, and the coefficient c of sqrt(t) = c ln s + 1
    rope_scale: float = 1.0
    rope_orig_ctx: int = 0
    yarn_alpha: float = 1.0
    yarn_beta: float = 32.0
    yarn_mscale: float = 0.0707
    # RMSNorm after the compressed latents c^q and c^KV (with learned gains), epsilon
    latent_norm: bool = False
    rms_eps: float = 1e-6

    @property
    def entry(self) -> int:
        """Values per cached token: [c_KV | k_R]."""
        return self.d_c + self.d_hr

    @property
    def q_in(self) -> int:
        """Input width of W_UQ / W_QR."""
        return self.d_cq if self.d_cq > 0 else self.d_model

    def weight_shapes(self) -> dict:
        s = {}
        if self.d_cq > 0:
            s["W_DQ"] = (self.d_cq, self.d_model)
        s["W_UQ"] = (self.n_h * self.d_h, self.q_in)
        s["W_QR"] = (self.n_h * self.d_hr, self.q_in)
        s["W_DKV"] = (self.d_c, self.d_model)
        s["W_KR"] = (self.d_hr, self.d_model)
        s["W_UK"] = (self.n_h * self.d_h, self.d_c)
        s["W_UV"] = (self.n_h * self.d_h, self.d_c)
        s["W_O"] = (self.d_model, self.n_h * self.d_h)
        return s

    def param_count(self) -> int:
        return int(sum(a * b for a, b in self.weight_shapes().values()))


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dims: Dims
    kind: str  # "decode" | "prefill" | "chunk" (ctx cached tokens, then a chunk of `tokens`)
    batch: int
    ctx: int = 0  # decode: tokens cached before the step (uniform contexts)
    ctx_lo: int = 0  # decode, ragged: lengths uniform in [ctx_lo, ctx_hi]
    ctx_hi: int = 0
    tokens: int = 0  # prefill: tokens per sequence
    decode_steps: int = 0  # prefill workloads that continue with decode steps
    block_size: int = 64
    hidden: str = "rmsnorm"  # "rmsnorm" (N(0,1) then RMS-normalised) | "normal002"
    weight_std: float = 0.02
    cache: str = "native"  # "native" (the dims' dtype) | "fp8" (per-token-scaled e4m3 codes)


TINY = Dims(d_model=64, n_h=4, d_h=16, d_c=32, d_cq=48, d_hr=8, dtype=F32)
V2_LITE = Dims(d_model=2048, n_h=16, d_h=128, d_c=512, d_cq=0, d_hr=64, dtype=BF16)
V2 = Dims(d_model=5120, n_h=128, d_h=128, d_c=512, d_cq=1536, d_hr=64, dtype=BF16)
# V2 with the long-context extension of section 3.1.4: s = 40 over a 4096-token original context
V2_YARN = dataclasses.replace(V2, rope_scale=40.0, rope_orig_ctx=4096)
TINY_YARN = dataclasses.replace(TINY, rope_scale=4.0, rope_orig_ctx=64)
# the layers with RMSNorm on the latents (section 3.1.2)
V2_NORM = dataclasses.replace(V2, latent_norm=True)
V2_LITE_NORM = dataclasses.replace(V2_LITE, latent_norm=True)
TINY_NORM = dataclasses.replace(TINY, latent_norm=True)

WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", TINY, "prefill", batch=1, tokens=16, decode_steps=4,
                          hidden="normal002"),
    "v2lite_decode_b8_ctx4096": Workload("v2lite_decode_b8_ctx4096", V2_LITE, "decode", batch=8,
                                         ctx=4096),
    "v2_decode_b64_ctx8192": Workload("v2_decode_b64_ctx8192", V2, "decode", batch=64, ctx=8192),
    "v2_decode_b64_ctx8192_fp8": Workload("v2_decode_b64_ctx8192_fp8", V2, "decode", batch=64, ctx=8192,
                                          cache="fp8"),
    # the same step with the latent RMSNorms (section 3.1.2) and YaRN (section 3.1.4) on
    "v2_decode_b64_ctx8192_norm_yarn": Workload("v2_decode_b64_ctx8192_norm_yarn",
                                                dataclasses.replace(V2_YARN, latent_norm=True), "decode",
                                                batch=64, ctx=8192),
    "v2_prefill_16384": Workload("v2_prefill_16384", V2, "prefill", batch=1, tokens=16384),
    # chunked prefill: the last 512 tokens of a 16384-token prompt after 15872 cached ones
    "v2_chunk_512_after_15872": Workload("v2_chunk_512_after_15872", V2, "chunk", batch=1, ctx=15872,
                                         tokens=512),
    "v2_long_decode_b4": Workload("v2_long_decode_b4", V2, "decode", batch=4, ctx_lo=32768,
                                  ctx_hi=131072),
}


# ----------------------------------------------------------------------------- rounding
def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 holding bf16 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Bit patterns (uint16) of an fp32 array whose values are bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> fp32 values."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values to the storage type; always returns fp32 holding exact values."""
    x = np.asarray(x, dtype=np.float32)
    return round_bf16(x) if dtype == BF16 else np.ascontiguousarray(x)


# ----------------------------------------------------------------------------- draws
def make_weights(dims: Dims, std: float = 0.02, seed: int = SEED_WEIGHTS) -> dict:
    """All weights, y = W x form, row-major [out][in], N(0, std) drawn in fp64 from one
    generator in WEIGHT_ORDER, cast to fp32 and rounded to the storage type."""
    rng = np.random.default_rng(seed)
    shapes = dims.weight_shapes()
    out = {}
    for name in WEIGHT_ORDER:
        if name not in shapes:
            continue
        w = rng.standard_normal(shapes[name]) * std
        out[name] = to_dtype(w.astype(np.float32), dims.dtype)
    if dims.latent_norm:  # norm gains 1 + N(0, 0.1), from their own generator
        g = np.random.default_rng(SEED_GAINS)
        if dims.d_cq > 0:
            out["g_cq"] = to_dtype((1.0 + 0.1 * g.standard_normal(dims.d_cq)).astype(np.float32), dims.dtype)
        out["g_ckv"] = to_dtype((1.0 + 0.1 * g.standard_normal(dims.d_c)).astype(np.float32), dims.dtype)
    return out


def _hidden_from(rng: np.random.Generator, n: int, d: int, recipe: str, dtype: str) -> np.ndarray:
    if recipe == "normal002":
        h = (rng.standard_normal((n, d)) * 0.02).astype(np.float32)
    elif recipe == "rmsnorm":
        h = rng.standard_normal((n, d), dtype=np.float32)
        ms = np.mean(np.square(h, dtype=np.float32), axis=1, keepdims=True, dtype=np.float32)
        h = h / np.sqrt(ms + np.float32(1e-6))
    elif recipe == "unit":
        h = rng.standard_normal((n, d)).astype(np.float32)
    else:
        raise ValueError(recipe)
    return to_dtype(h, dtype)


def hidden_history(dims: Dims, seq: int, n: int, recipe: str, seed: int = SEED_HISTORY) -> np.ndarray:
    """Hidden states of the first n tokens of sequence `seq`; each sequence has its own
    generator, so any sequence can be regenerated on its own."""
    return _hidden_from(np.random.default_rng([seed, seq]), n, dims.d_model, recipe, dims.dtype)


def hidden_histories(dims: Dims, lens, recipe: str, seed: int = SEED_HISTORY, threads: int = 0):
    """hidden_history for sequences 0..len(lens)-1 in parallel threads (numpy's
    generators release the GIL)."""
    threads = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(max(1, threads)) as ex:
        return list(ex.map(lambda b: hidden_history(dims, b, int(lens[b]), recipe, seed), range(len(lens))))


def hidden_step(dims: Dims, batch: int, recipe: str, step: int = 0, seed: int = SEED_STEP) -> np.ndarray:
    """Hidden states [batch, d_model] of the token decoded at step `step`."""
    return _hidden_from(np.random.default_rng([seed, step]), batch, dims.d_model, recipe, dims.dtype)


def page_permutation(num_blocks: int, seed: int = SEED_PAGES) -> np.ndarray:
    """Physical block ids in a seeded random order (int32)."""
    return np.random.default_rng(seed).permutation(num_blocks).astype(np.int32)


def ragged_lengths(batch: int, lo: int, hi: int, seed: int = SEED_LENGTHS) -> np.ndarray:
    """Context lengths uniform on the integers [lo, hi] (int64)."""
    return np.random.default_rng(seed).integers(lo, hi + 1, size=batch).astype(np.int64)


def context_lengths(w: Workload) -> np.ndarray:
    if w.ctx_hi > 0:
        return ragged_lengths(w.batch, w.ctx_lo, w.ctx_hi)
    return np.full(w.batch, w.ctx, dtype=np.int64)


def block_table(lens_plus_new, block_size: int, seed: int = SEED_PAGES):
    """Block table [batch][max_blocks] (int32) mapping every sequence's logical pages to a
    seeded permutation of the pool's physical pages; returns (table, num_blocks)."""
    nblk = [(int(n) + block_size - 1) // block_size for n in lens_plus_new]
    total = int(sum(nblk))
    perm = page_permutation(max(total, 1), seed)
    mx = max(max(nblk), 1)
    table = np.zeros((len(nblk), mx), dtype=np.int32)
    o = 0
    for b, k in enumerate(nblk):
        table[b, :k] = perm[o:o + k]
        o += k
    return table, max(total, 1)


# ----------------------------------------------------------------------------- fp8 cache inputs
SEED_FP8 = 5


def fp8_codes(n: int, entry: int, seed: int = SEED_FP8) -> np.ndarray:
    """Random e4m3 codes [n, entry] (uint8): random sign, exponent field 3..13, random mantissa,
    about 2% zero codes; never the NaN codes."""
    rng = np.random.default_rng(seed)
    sign = rng.integers(0, 2, (n, entry)) << 7
    e = rng.integers(3, 14, (n, entry)) << 3
    m = rng.integers(0, 8, (n, entry))
    codes = (sign | e | m).astype(np.uint8)
    codes[rng.random((n, entry)) < 0.02] = 0
    return codes


def fp8_scales(n: int, seed: int = SEED_FP8 + 1) -> np.ndarray:
    """Per-token (s_c, s_r) [n, 2] fp32: log-uniform in [2^-9, 2^-5], a few zero (all-zero parts)."""
    rng = np.random.default_rng(seed)
    s = np.exp2(rng.uniform(-9.0, -5.0, (n, 2))).astype(np.float32)
    s[rng.random((n, 2)) < 0.01] = 0.0
    return s


def quantizer_rows(n: int, entry: int, d_c: int, seed: int = SEED_FP8 + 2) -> np.ndarray:
    """bf16-exact rows [n, entry] for the fp8 quantiser: normal values at a per-row magnitude
    10^U(-4, 2), with some all-zero parts, single outliers, and values spread down into the
    subnormal range of the codes."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, entry)) * np.power(10.0, rng.uniform(-4, 2, (n, 1)))
    x[0] = 0.0
    if n > 1:
        x[1, :d_c] = 0.0
    if n > 2:
        x[2, d_c:] = 0.0
    for r in range(3, n, 7):
        x[r, rng.integers(0, entry)] *= 1e3          # one outlier: everything else small
    for r in range(5, n, 11):
        x[r] *= np.exp2(rng.uniform(-14, 0, entry))  # wide dynamic range within the row
    return round_bf16(x.astype(np.float32))
