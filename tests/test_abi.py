"""C ABI checks that need no GPU: the library loads, exports every entry point the header
declares, and rejects invalid arguments on the host before anything is launched."""
import ctypes
import os
import re

import pytest

import mla_latent_kv_27_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = M.lib()
    names = _declared()
    assert set(names) == set(M.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in (0, -1, -2, -3, -4):
        assert M.status_string(s).startswith("MLA_")
    assert "unknown" in M.status_string(7)


def _dims(**kw):
    base = dict(d_model=64, n_h=4, d_h=16, d_c=32, d_cq=48, d_hr=8, dtype="f32")
    base.update(kw)
    return M.make_dims(**base)


@pytest.mark.parametrize("bad", [dict(d_model=0), dict(n_h=-1), dict(d_hr=7), dict(d_c=0), dict(d_cq=-4),
                                 dict(rope_base=0.0), dict(softmax_scale=-1.0),
                                 dict(rope_scale=-1.0), dict(rope_scale=float("nan")),
                                 dict(rope_scale=40.0, rope_orig_ctx=0),
                                 dict(rope_scale=40.0, rope_orig_ctx=4096, yarn_alpha=32.0, yarn_beta=32.0),
                                 dict(rope_scale=40.0, rope_orig_ctx=4096, yarn_alpha=-1.0),
                                 dict(rope_scale=40.0, rope_orig_ctx=4096, yarn_mscale=-0.1),
                                 dict(rms_eps=-1e-6), dict(rms_eps=float("inf"))])
def test_invalid_dims_rejected(bad):
    out = ctypes.c_size_t(0)
    st = M.lib().mla_workspace_size(ctypes.byref(_dims(**bad)), M.OP_DECODE, 1, 0, 4, 0, ctypes.byref(out))
    assert st == M.MLA_ERR_INVALID_ARG


def test_yarn_off_values_accepted():
    # a scale of at most 1 turns YaRN off whatever the other fields hold
    out = ctypes.c_size_t(0)
    for kw in (dict(rope_scale=0.0), dict(rope_scale=1.0, rope_orig_ctx=-5, yarn_beta=-1.0),
               dict(rope_scale=40.0, rope_orig_ctx=4096)):
        st = M.lib().mla_workspace_size(ctypes.byref(_dims(**kw)), M.OP_DECODE, 1, 0, 4, 0, ctypes.byref(out))
        assert st == M.MLA_OK, kw


def test_unaligned_dims_unsupported():
    out = ctypes.c_size_t(0)
    st = M.lib().mla_workspace_size(ctypes.byref(_dims(d_model=66)), M.OP_DECODE, 1, 0, 4, 0, ctypes.byref(out))
    assert st == M.MLA_ERR_UNSUPPORTED


def _fake(n):
    return ctypes.c_void_p(0x1000 * n)


def _weights(dq=True, g_cq=None, g_ckv=None):
    return M.Weights(*([_fake(1) if dq else None] + [_fake(i) for i in range(2, 9)] + [g_cq, g_ckv]))


def _cache(num_blocks=4, block=64, maxb=2):
    return M.PagedCache(_fake(20), num_blocks, block, maxb, _fake(21))


def _decode(dims=None, w=None, c=None, h=_fake(30), batch=2, ctx=_fake(31), max_ctx=10, splits=0, u=_fake(32),
            ws=None, ws_bytes=0):
    dims = dims or _dims()
    w = w or _weights()
    c = c or _cache()
    return M.lib().mla_decode(ctypes.byref(dims), ctypes.byref(w), ctypes.byref(c), h, batch, ctx, max_ctx, splits,
                              u, None, ws, ws_bytes, None)


def test_decode_host_validation():
    assert _decode(h=None) == M.MLA_ERR_INVALID_ARG
    assert _decode(u=None) == M.MLA_ERR_INVALID_ARG
    assert _decode(ctx=None) == M.MLA_ERR_INVALID_ARG
    assert _decode(batch=0) == M.MLA_ERR_INVALID_ARG
    assert _decode(splits=-1) == M.MLA_ERR_INVALID_ARG
    # W_DQ must be present iff d_cq > 0
    assert _decode(w=_weights(dq=False)) == M.MLA_ERR_INVALID_ARG
    assert _decode(dims=_dims(d_cq=0)) == M.MLA_ERR_INVALID_ARG
    # the c^q norm needs query compression; the c^KV norm does not
    assert _decode(dims=_dims(d_cq=0), w=_weights(dq=False, g_cq=_fake(50))) == M.MLA_ERR_INVALID_ARG
    assert _decode(dims=_dims(d_cq=0), w=_weights(dq=False, g_ckv=_fake(51)), max_ctx=127) == M.MLA_ERR_WORKSPACE
    assert _decode(w=_weights(g_cq=_fake(50), g_ckv=_fake(51)), max_ctx=127) == M.MLA_ERR_WORKSPACE
    # ctx_len + 1 must fit in max_blocks_per_seq * block_size (2 * 64)
    assert _decode(max_ctx=128) == M.MLA_ERR_INVALID_ARG
    # no cache pool
    assert _decode(c=M.PagedCache(None, 4, 64, 2, _fake(21))) == M.MLA_ERR_INVALID_ARG
    assert _decode(c=M.PagedCache(_fake(20), 4, 0, 2, _fake(21))) == M.MLA_ERR_INVALID_ARG
    # sizes without a decode kernel
    assert _decode(dims=_dims(d_c=64)) == M.MLA_ERR_UNSUPPORTED
    # valid arguments but no workspace
    assert _decode(max_ctx=127) == M.MLA_ERR_WORKSPACE
    assert _decode(max_ctx=127, ws=_fake(40), ws_bytes=16) == M.MLA_ERR_WORKSPACE


def test_prefill_and_append_host_validation():
    L = M.lib()
    d, w, c = _dims(), _weights(), _cache()
    P = ctypes.byref
    assert L.mla_prefill(P(d), P(w), P(c), None, 1, 16, _fake(2), None, None, 0, None) == M.MLA_ERR_INVALID_ARG
    assert L.mla_prefill(P(d), P(w), P(c), _fake(1), 1, 0, _fake(2), None, None, 0, None) == M.MLA_ERR_INVALID_ARG
    assert L.mla_prefill(P(d), P(w), P(c), _fake(1), 1, 129, _fake(2), None, None, 0, None) == M.MLA_ERR_INVALID_ARG
    assert L.mla_prefill(P(d), P(w), P(c), _fake(1), 1, 16, _fake(2), None, None, 0, None) == M.MLA_ERR_WORKSPACE
    assert L.mla_cache_append(P(d), P(w), P(c), None, 4, _fake(3), _fake(4), None, 0, None) == M.MLA_ERR_INVALID_ARG
    assert L.mla_cache_append(P(d), P(w), P(c), _fake(1), -1, _fake(3), _fake(4), None, 0, None) == M.MLA_ERR_INVALID_ARG
    assert L.mla_cache_append(P(d), P(w), P(c), _fake(1), 0, None, None, None, 0, None) == M.MLA_OK
    assert L.mla_cache_append(P(d), P(w), P(c), _fake(1), 4, _fake(3), _fake(4), None, 0, None) == M.MLA_ERR_WORKSPACE
    assert L.mla_decode_attention(P(d), P(c), _fake(1), 2, _fake(2), 0, 0, _fake(3), None, None, 0,
                                  None) == M.MLA_ERR_INVALID_ARG


def test_prefill_chunk_host_validation():
    L = M.lib()
    d, w, c = _dims(), _weights(), _cache()  # capacity 2 blocks x 64 tokens
    P = ctypes.byref

    def chunk(start=_fake(5), max_start=10, T=16, ws=None, ws_bytes=0):
        return L.mla_prefill_chunk(P(d), P(w), P(c), _fake(1), 1, T, start, max_start, _fake(2), None, ws, ws_bytes,
                                   None)
    assert chunk(start=None) == M.MLA_ERR_INVALID_ARG
    assert chunk(max_start=-1) == M.MLA_ERR_INVALID_ARG
    assert chunk(max_start=113) == M.MLA_ERR_INVALID_ARG  # 113 + 16 > 128
    assert chunk(max_start=112) == M.MLA_ERR_WORKSPACE
    out = ctypes.c_size_t(0)
    assert L.mla_workspace_size(P(d), M.OP_PREFILL_CHUNK, 1, 16, -1, 0, P(out)) == M.MLA_ERR_INVALID_ARG
    sizes = []
    for ms in (0, 100, 1000):
        assert L.mla_workspace_size(P(d), M.OP_PREFILL_CHUNK, 2, 16, ms, 0, P(out)) == M.MLA_OK
        sizes.append(out.value)
    assert sizes[0] < sizes[1] < sizes[2]


def test_workspace_sizes_grow_with_work():
    d = _dims()
    a = M.workspace_size(d, M.OP_DECODE, batch=2, max_ctx_len=100)
    b = M.workspace_size(d, M.OP_DECODE, batch=8, max_ctx_len=100)
    assert 0 < a < b
    p1 = M.workspace_size(d, M.OP_PREFILL, batch=1, max_tokens=16)
    p2 = M.workspace_size(d, M.OP_PREFILL, batch=2, max_tokens=64)
    assert 0 < p1 < p2
    with pytest.raises(M.MlaError):
        M.workspace_size(d, 9)


def test_workspace_for_max_sizes_serves_every_smaller_call():
    """A workspace sized for (n, batch, context) also fits every call with smaller sizes."""
    d = M.make_dims(5120, 128, 128, 512, 1536, 64, "bf16")
    big = M.workspace_size(d, M.OP_CACHE_APPEND, max_tokens=8192)
    assert all(M.workspace_size(d, M.OP_CACHE_APPEND, max_tokens=n) <= big for n in range(1, 8193, 97))
    big = M.workspace_size(d, M.OP_DECODE, batch=64, max_ctx_len=8192)
    for b in (1, 3, 5, 6, 17, 63, 64):
        for ctx in (0, 100, 4095, 8192):
            assert M.workspace_size(d, M.OP_DECODE, batch=b, max_ctx_len=ctx) <= big, (b, ctx)
    big = M.workspace_size(d, M.OP_DECODE, batch=4, max_ctx_len=131072, num_splits=7)
    for ctx in (1, 700, 22 * 32, 21 * 32, 131071):
        assert M.workspace_size(d, M.OP_DECODE, batch=4, max_ctx_len=ctx, num_splits=7) <= big


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define MLA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == M.NOALLOC_SCRATCH_BYTES
    # the DeepSeek-V2 decode sizes the header promises fit
    d = M.make_dims(5120, 128, 128, 512, 1536, 64, "bf16")
    for B, ctx in ((64, 131072), (64, 8192), (4, 131072), (1, 131072)):
        assert M.workspace_size(d, M.OP_DECODE, batch=B, max_ctx_len=ctx) <= M.NOALLOC_SCRATCH_BYTES, (B, ctx)
