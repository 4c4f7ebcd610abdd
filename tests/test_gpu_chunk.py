"""GPU parity of chunked prefill (mla_prefill_chunk: the next T tokens of sequences whose first
start_pos[b] tokens are cached; App. C's causal sum over the prefix and the chunk) through the C
ABI, against the oracle's prefill with a prefix (pinned in test_oracle.py: chunked prefill equals
the whole), on V2 with ragged prefixes, the fp32 tiny layer chunk by chunk, the fp8 cache (the
prefix read back dequantised), and the layer with the latent norms and YaRN on."""
import dataclasses

import numpy as np
import pytest

import mla_synth as S
import oracle.latent_fp8 as F
import oracle.mla_oracle as O
from tests.gpu_util import check, have_gpu, torch

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

import mla_latent_kv_27_amd as M  # noqa: E402
from mla_latent_kv_27_amd import workload as WL  # noqa: E402


def _chunk(layer, pool, hs_chunk, starts, o_heads=True):
    dims = layer.dims
    B, T = hs_chunk.shape[0], hs_chunk.shape[1]
    u = torch.empty((B, T, dims.d_model), dtype=WL.torch_dtype(dims), device="cuda")
    oh = torch.empty((B, T, dims.n_h, dims.d_h), dtype=torch.float32, device="cuda") if o_heads else None
    st = torch.tensor(starts, dtype=torch.int32, device="cuda")
    M.prefill_chunk(layer.cdims, layer.cweights, pool.ccache, WL.to_device(hs_chunk, dims), st, max(starts), u,
                    WL.chunk_workspace(layer, B, T, max(starts)), o_heads=oh)
    torch.cuda.synchronize()
    return u, oh


@pytest.mark.parametrize("dims,prefixes,T", [(S.V2, [100, 257], 64), (S.V2, [0, 31], 130),
                                             (dataclasses.replace(S.V2_YARN, latent_norm=True), [300, 4500], 40)])
def test_chunk_after_cached_prefix(dims, prefixes, T):
    W = S.make_weights(dims)
    layer = WL.DeviceLayer(dims, W)
    B = len(prefixes)
    pool = WL.PagedPool(dims, [p + T for p in prefixes])
    WL.build_context(layer, pool, prefixes, "rmsnorm")
    hist = [S.hidden_history(dims, b, p + T, "rmsnorm") for b, p in enumerate(prefixes)]
    u, oh = _chunk(layer, pool, np.stack([h[p:] for h, p in zip(hist, prefixes)]), prefixes)
    for b, p in enumerate(prefixes):
        prefix = pool.read_entries(b, p) if p else None
        ref = O.mla_prefill(W, dims, hist[b][p:], start_pos=p, prefix_cache=prefix)
        check(pool.read_entries(b, p + T)[p:], ref["cache"][p:], dims.dtype, f"chunk cache b={b}")
        check(oh[b].cpu().numpy(), ref["o"], dims.dtype, f"chunk o b={b}")
        check(u[b].float().cpu().numpy(), ref["u"], dims.dtype, f"chunk u b={b}")


def test_tiny_chunks_equal_whole_prefill():
    """fp32 tiny layer: 40 tokens in chunks of 7 (the last one ragged in its page) equal the
    oracle's prefill of all 40."""
    dims = S.TINY
    W = S.make_weights(dims)
    layer = WL.DeviceLayer(dims, W)
    h = S.hidden_history(dims, 0, 40, "normal002")
    pool = WL.PagedPool(dims, [40], block_size=4)
    ref = O.mla_prefill(W, dims, h)
    for s0 in range(0, 40, 7):
        T = min(7, 40 - s0)
        u, oh = _chunk(layer, pool, h[None, s0:s0 + T], [s0])
        check(u[0].cpu().numpy(), ref["u"][s0:s0 + T], dims.dtype, f"tiny chunk at {s0} u")
        check(oh[0].cpu().numpy(), ref["o"][s0:s0 + T], dims.dtype, f"tiny chunk at {s0} o")
    check(pool.read_entries(0, 40), ref["cache"], dims.dtype, "tiny chunked cache")


def test_chunk_from_zero_equals_prefill():
    dims = S.V2
    layer = WL.DeviceLayer(dims, S.make_weights(dims))
    T = 97
    h = np.stack([S.hidden_history(dims, b, T, "rmsnorm") for b in range(2)])
    pool_a, pool_b = WL.PagedPool(dims, [T, T]), WL.PagedPool(dims, [T, T])
    ua = torch.empty((2, T, dims.d_model), dtype=torch.bfloat16, device="cuda")
    M.prefill(layer.cdims, layer.cweights, pool_a.ccache, WL.to_device(h, dims), ua, WL.prefill_workspace(layer, 2, T))
    ub, _ = _chunk(layer, pool_b, h, [0, 0], o_heads=False)
    check(ub.float().cpu().numpy(), ua.float().cpu().numpy(), dims.dtype, "chunk from 0 vs prefill")
    assert np.array_equal(pool_a.read_entries(1, T), pool_b.read_entries(1, T))


def test_fp8_cache_prefix_is_read_dequantised():
    dims = S.V2
    W = S.make_weights(dims)
    layer = WL.DeviceLayer(dims, W, cache_dtype="fp8")
    prefixes, T = [200, 77], 48
    pool = WL.PagedPool(dims, [p + T for p in prefixes], fp8=True)
    WL.build_context(layer, pool, prefixes, "rmsnorm")
    hist = [S.hidden_history(dims, b, p + T, "rmsnorm") for b, p in enumerate(prefixes)]
    u, oh = _chunk(layer, pool, np.stack([h[p:] for h, p in zip(hist, prefixes)]), prefixes)
    for b, p in enumerate(prefixes):
        codes, scales = pool.read_codes(b, p)
        ref = O.mla_prefill(W, dims, hist[b][p:], start_pos=p, prefix_cache=F.dequantize(codes, scales, dims.d_c))
        check(oh[b].cpu().numpy(), ref["o"], dims.dtype, f"fp8 chunk o b={b}")
        check(u[b].float().cpu().numpy(), ref["u"], dims.dtype, f"fp8 chunk u b={b}")
        new_codes, _ = pool.read_codes(b, p + T)
        ref_codes, _ = F.quantize_entries(F.bf16_round(ref["cache"][p:]), dims.d_c)
        assert np.mean(new_codes[p:] == ref_codes) >= 0.99, b
