"""Python binding of libmla (MI355X / gfx950 Multi-head Latent Attention).

Argument marshalling only: every step of the computation runs in the HIP kernels behind the
C ABI declared in include/mla.h.  torch supplies device memory and streams.  There is no
fallback path: if the library is missing or fails to load, importing the binding's entry
points raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# MLA_LIBRARY selects another build of the same library (the debug or sanitizer variants that
# build.py makes beside it); the default is the release build
LIB_PATH = os.environ.get("MLA_LIBRARY") or os.path.join(PKG, "lib", "libmla.so")

MLA_OK = 0
MLA_ERR_INVALID_ARG = -1
MLA_ERR_UNSUPPORTED = -2
MLA_ERR_WORKSPACE = -3
MLA_ERR_HIP = -4
MLA_F32 = 0
MLA_BF16 = 1
MLA_FP8_E4M3 = 2
OP_CACHE_APPEND, OP_PREFILL, OP_DECODE, OP_PREFILL_CHUNK = 0, 1, 2, 3

EXPORTED = (
    "mla_workspace_size", "mla_cache_append", "mla_prefill", "mla_prefill_chunk", "mla_decode", "mla_decode_noalloc",
    "mla_decode_attention", "mla_decode_attention_partials", "mla_decode_auto_splits", "mla_quantize_entries",
    "mla_status_string",
)
# bytes of the library's own scratch behind mla_decode_noalloc (MLA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 192 << 20


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class Dims(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_h", ctypes.c_int32), ("d_h", ctypes.c_int32),
                ("d_c", ctypes.c_int32), ("d_cq", ctypes.c_int32), ("d_hr", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("rope_base", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("cache_dtype", ctypes.c_int32), ("rope_scale", ctypes.c_float), ("rope_orig_ctx", ctypes.c_int32),
                ("yarn_alpha", ctypes.c_float), ("yarn_beta", ctypes.c_float), ("yarn_mscale", ctypes.c_float),
                ("rms_eps", ctypes.c_float)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("W_DQ", "W_UQ", "W_QR", "W_DKV", "W_KR", "W_UK", "W_UV", "W_O",
                                                "g_cq", "g_ckv")]


class PagedCache(ctypes.Structure):
    _fields_ = [("pool", ctypes.c_void_p), ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("block_table", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmla.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmla.so not found at {LIB_PATH}; build it with "
                               "`python -m mla_latent_kv_27_amd.build` (there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        D, W, C = ctypes.POINTER(Dims), ctypes.POINTER(Weights), ctypes.POINTER(PagedCache)
        L.mla_workspace_size.argtypes = [D, ctypes.c_int, I32, I32, I32, I32, ctypes.POINTER(SZ)]
        L.mla_cache_append.argtypes = [D, W, C, P, I32, P, P, P, SZ, P]
        L.mla_prefill.argtypes = [D, W, C, P, I32, I32, P, P, P, SZ, P]
        L.mla_prefill_chunk.argtypes = [D, W, C, P, I32, I32, P, I32, P, P, P, SZ, P]
        L.mla_decode.argtypes = [D, W, C, P, I32, P, I32, I32, P, P, P, SZ, P]
        L.mla_decode_noalloc.argtypes = [D, W, C, P, I32, P, I32, I32, P, P, P]
        L.mla_decode_attention.argtypes = [D, C, P, I32, P, I32, I32, P, P, P, SZ, P]
        L.mla_decode_attention_partials.argtypes = [D, C, P, I32, P, I32, I32, P, P, P, ctypes.POINTER(I32), P]
        L.mla_decode_auto_splits.argtypes = [D, I32, I32]
        L.mla_quantize_entries.argtypes = [D, P, I32, P, P, P]
        L.mla_quantize_entries.restype = ctypes.c_int
        L.mla_decode_auto_splits.restype = I32
        L.mla_status_string.argtypes = [ctypes.c_int]
        L.mla_status_string.restype = ctypes.c_char_p
        for n in ("mla_workspace_size", "mla_cache_append", "mla_prefill", "mla_prefill_chunk", "mla_decode",
                  "mla_decode_noalloc", "mla_decode_attention", "mla_decode_attention_partials"):
            getattr(L, n).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().mla_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != MLA_OK:
        raise MlaError(status, where)


def _ptr(t) -> int | None:
    """Device (or host) address of a tensor, or None."""
    if t is None:
        return None
    return int(t.data_ptr())


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream) or None
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def make_dims(d_model, n_h, d_h, d_c, d_cq, d_hr, dtype, softmax_scale=0.0, rope_base=10000.0,
              cache_dtype=0, rope_scale=1.0, rope_orig_ctx=0, yarn_alpha=1.0, yarn_beta=32.0,
              yarn_mscale=0.0707, rms_eps=0.0) -> Dims:
    """YaRN is on when rope_scale > 1 (then rope_orig_ctx > 0 is required); rms_eps 0 = 1e-6."""
    dt = {"bf16": MLA_BF16, "f32": MLA_F32, MLA_BF16: MLA_BF16, MLA_F32: MLA_F32}[dtype]
    cdt = {0: 0, None: 0, "fp8": MLA_FP8_E4M3, MLA_FP8_E4M3: MLA_FP8_E4M3}[cache_dtype]
    return Dims(d_model, n_h, d_h, d_c, d_cq, d_hr, float(softmax_scale), float(rope_base), dt, cdt,
                float(rope_scale), int(rope_orig_ctx), float(yarn_alpha), float(yarn_beta), float(yarn_mscale),
                float(rms_eps))


def make_weights(W: dict) -> Weights:
    """W maps the names W_DQ .. W_O (and the optional norm gains g_cq, g_ckv) to device tensors
    (W_DQ and the gains may be absent)."""
    return Weights(*[_ptr(W.get(n)) for n, _ in Weights._fields_])


def make_cache(pool, block_table, scales=None) -> PagedCache:
    """pool [num_blocks][block_size][d_c + d_hr], block_table [batch][max_blocks] int32;
    scales [num_blocks][block_size][2] fp32 for an fp8 cache."""
    return PagedCache(_ptr(pool), pool.shape[0], pool.shape[1], block_table.shape[1], _ptr(block_table),
                      _ptr(scales))


def workspace_size(dims: Dims, op: int, batch: int = 0, max_tokens: int = 0, max_ctx_len: int = 0,
                   num_splits: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().mla_workspace_size(ctypes.byref(dims), op, batch, max_tokens, max_ctx_len, num_splits,
                                    ctypes.byref(out)), "mla_workspace_size")
    return out.value


def _ws(ws):
    return (_ptr(ws), 0 if ws is None else ws.numel() * ws.element_size())


def cache_append(dims, weights, cache, h, seq_idx, pos, workspace, stream=None):
    p, n = _ws(workspace)
    _check(lib().mla_cache_append(ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(cache), _ptr(h),
                                  int(h.shape[0]), _ptr(seq_idx), _ptr(pos), p, n, _stream(stream)),
           "mla_cache_append")


def prefill(dims, weights, cache, h, u, workspace, o_heads=None, stream=None):
    """h, u: [batch][T][d_model]."""
    p, n = _ws(workspace)
    _check(lib().mla_prefill(ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(cache), _ptr(h),
                             int(h.shape[0]), int(h.shape[1]), _ptr(u), _ptr(o_heads), p, n, _stream(stream)),
           "mla_prefill")


def prefill_chunk(dims, weights, cache, h, start_pos, max_start, u, workspace, o_heads=None, stream=None):
    """h, u: [batch][T][d_model]; start_pos: int32 device tensor [batch] of tokens already cached."""
    p, n = _ws(workspace)
    _check(lib().mla_prefill_chunk(ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(cache), _ptr(h),
                                   int(h.shape[0]), int(h.shape[1]), _ptr(start_pos), int(max_start), _ptr(u),
                                   _ptr(o_heads), p, n, _stream(stream)), "mla_prefill_chunk")


def decode(dims, weights, cache, h, ctx_lens, max_ctx_len, u, workspace, num_splits=0, o_heads=None,
           stream=None):
    p, n = _ws(workspace)
    _check(lib().mla_decode(ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(cache), _ptr(h),
                            int(h.shape[0]), _ptr(ctx_lens), int(max_ctx_len), int(num_splits), _ptr(u),
                            _ptr(o_heads), p, n, _stream(stream)), "mla_decode")


def decode_noalloc(dims, weights, cache, h, ctx_lens, max_ctx_len, u, num_splits=0, o_heads=None, stream=None):
    """mla_decode on the library's own scratch (no workspace; see mla_decode_noalloc in mla.h)."""
    _check(lib().mla_decode_noalloc(ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(cache), _ptr(h),
                                    int(h.shape[0]), _ptr(ctx_lens), int(max_ctx_len), int(num_splits), _ptr(u),
                                    _ptr(o_heads), _stream(stream)), "mla_decode_noalloc")


def decode_attention(dims, cache, q, kv_lens, max_kv_len, o_hat, workspace, num_splits=0, lse=None,
                     stream=None):
    p, n = _ws(workspace)
    _check(lib().mla_decode_attention(ctypes.byref(dims), ctypes.byref(cache), _ptr(q), int(q.shape[0]),
                                      _ptr(kv_lens), int(max_kv_len), int(num_splits), _ptr(o_hat), _ptr(lse),
                                      p, n, _stream(stream)), "mla_decode_attention")


def decode_attention_partials(dims, cache, q, kv_lens, max_kv_len, num_splits, part_m, part_l, part_o,
                              stream=None) -> int:
    """The attention core's per-partition (max, sum, normalised output) without their reduction;
    buffers sized for num_splits partitions; returns the number of partitions P."""
    out = ctypes.c_int32(0)
    _check(lib().mla_decode_attention_partials(ctypes.byref(dims), ctypes.byref(cache), _ptr(q), int(q.shape[0]),
                                               _ptr(kv_lens), int(max_kv_len), int(num_splits), _ptr(part_m),
                                               _ptr(part_l), _ptr(part_o), ctypes.byref(out), _stream(stream)),
           "mla_decode_attention_partials")
    return int(out.value)


def quantize_entries(dims, entries, codes, scales, stream=None):
    """entries [n][d_c + d_hr] bf16 -> codes [n][d_c + d_hr] uint8, scales [n][2] fp32."""
    _check(lib().mla_quantize_entries(ctypes.byref(dims), _ptr(entries), int(entries.shape[0]), _ptr(codes),
                                      _ptr(scales), _stream(stream)), "mla_quantize_entries")


def auto_splits(dims, batch, max_ctx_len) -> int:
    return int(lib().mla_decode_auto_splits(ctypes.byref(dims), int(batch), int(max_ctx_len)))
