"""mla_decode_noalloc (the decode step on the library's own scratch, for callers that cannot
allocate) against mla_decode with a caller workspace: two calls in a row through the C ABI, the
second with a smaller batch and shorter contexts, must give the same u and per-head o bit for bit
(the same kernels on the same inputs), and a call whose sizes need more scratch than the library
holds is refused."""
import numpy as np
import pytest

import mla_synth as S
from tests.gpu_util import have_gpu

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs an MI355X")]

import mla_latent_kv_27_amd as M  # noqa: E402
from mla_latent_kv_27_amd import workload as WL  # noqa: E402


def _both(layer, pool, lens, step):
    dims = layer.dims
    B = len(lens)
    h = WL.to_device(S.hidden_step(dims, B, "rmsnorm", step=step), dims)
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    mx = int(max(lens))
    u_ws = torch.full((B, dims.d_model), float("nan"), dtype=WL.torch_dtype(dims), device="cuda")
    u_na = torch.full_like(u_ws, float("nan"))
    o_ws = torch.full((B, dims.n_h, dims.d_h), float("nan"), dtype=torch.float32, device="cuda")
    o_na = torch.full_like(o_ws, float("nan"))
    # the new entry is rewritten at the same slot by both calls (same values)
    M.decode(layer.cdims, layer.cweights, pool.ccache, h, ctx, mx, u_ws, WL.decode_workspace(layer, B, mx),
             o_heads=o_ws)
    M.decode_noalloc(layer.cdims, layer.cweights, pool.ccache, h, ctx, mx, u_na, o_heads=o_na)
    torch.cuda.synchronize()
    return u_ws, u_na, o_ws, o_na


@pytest.mark.parametrize("name", ["v2", "v2lite"])
def test_noalloc_decode_equals_workspace_decode_two_calls(name):
    dims = S.V2 if name == "v2" else S.V2_LITE
    layer = WL.DeviceLayer(dims, S.make_weights(dims))
    first, second = [700, 129, 1000, 64, 333, 5], [150, 3]
    pool = WL.PagedPool(dims, [L + 1 for L in first], block_size=64)
    WL.build_context(layer, pool, first, "rmsnorm")
    for step, lens in enumerate((first, second)):
        u_ws, u_na, o_ws, o_na = _both(layer, pool, lens, step)
        assert torch.isfinite(u_ws.float()).all() and torch.isfinite(o_ws).all()
        assert torch.equal(u_na, u_ws), f"call {step}: u differs"
        assert torch.equal(o_na, o_ws), f"call {step}: o differs"


def test_noalloc_refuses_sizes_beyond_its_scratch():
    dims = S.V2
    layer = WL.DeviceLayer(dims, S.make_weights(dims))
    B = 1024  # the workspace of 1024 sequences exceeds the library's scratch
    assert M.workspace_size(layer.cdims, M.OP_DECODE, batch=B, max_ctx_len=64) > M.NOALLOC_SCRATCH_BYTES
    pool = WL.PagedPool(dims, [65] * 2, block_size=64)
    h = torch.zeros((B, dims.d_model), dtype=torch.bfloat16, device="cuda")
    ctx = torch.zeros(B, dtype=torch.int32, device="cuda")
    u = torch.zeros((B, dims.d_model), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(M.MlaError) as e:
        M.decode_noalloc(layer.cdims, layer.cweights, pool.ccache, h, ctx, 64, u)
    assert e.value.status == M.MLA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert not u.any()  # nothing was launched
