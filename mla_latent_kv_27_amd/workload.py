"""Device-side set-up of synthetic MLA workloads: weights, paged pools, block tables and decode
contexts built through the library's own cache writer.  Used by the GPU tests, the smoke check
and the benchmark.  Inputs come from the seeded generators in `mla_synth`.
"""
from __future__ import annotations

import numpy as np
import torch

import mla_synth as S

from . import (OP_CACHE_APPEND, OP_DECODE, OP_PREFILL, OP_PREFILL_CHUNK, cache_append, make_cache, make_dims, make_weights,
               workspace_size)


def torch_dtype(dims: S.Dims):
    return torch.bfloat16 if dims.dtype == S.BF16 else torch.float32


def to_device(x: np.ndarray, dims: S.Dims, device="cuda") -> torch.Tensor:
    """fp32 array holding values exact in the storage type -> device tensor of that type."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device=device, dtype=torch_dtype(dims))


class DeviceLayer:
    """One MLA layer's weights on the device plus the C structs describing them."""

    def __init__(self, dims: S.Dims, W_np: dict, device="cuda", cache_dtype=0):
        """cache_dtype: 0 (the layer's dtype) or "fp8" (per-token-scaled e4m3 cache)."""
        self.dims = dims
        self.device = device
        self.W = {k: to_device(v, dims, device) for k, v in W_np.items()}
        self.cdims = make_dims(dims.d_model, dims.n_h, dims.d_h, dims.d_c, dims.d_cq, dims.d_hr, dims.dtype,
                               dims.softmax_scale, dims.rope_base, cache_dtype, rope_scale=dims.rope_scale,
                               rope_orig_ctx=dims.rope_orig_ctx, yarn_alpha=dims.yarn_alpha,
                               yarn_beta=dims.yarn_beta, yarn_mscale=dims.yarn_mscale, rms_eps=dims.rms_eps)
        self.cweights = make_weights(self.W)

    def clone(self) -> "DeviceLayer":
        c = DeviceLayer.__new__(DeviceLayer)
        c.dims, c.device, c.cdims = self.dims, self.device, self.cdims
        c.W = {k: v.clone() for k, v in self.W.items()}
        c.cweights = make_weights(c.W)
        return c


class PagedPool:
    """A paged latent cache with a seeded random page permutation.  capacity[b] = tokens that
    sequence b may hold.  Unused slots are filled with `fill` (NaN by default, so that a read of
    a slot outside a context shows up in the outputs)."""

    def __init__(self, dims: S.Dims, capacity, block_size=64, device="cuda", fill=float("nan"), seed=S.SEED_PAGES,
                 fp8=False):
        """fp8: the pool holds e4m3 codes (unused slots 0x7F, a NaN code) with per-token scales."""
        table, nblk = S.block_table(capacity, block_size, seed)
        self.dims = dims
        self.block_size = block_size
        self.fp8 = fp8
        if fp8:
            self.pool = torch.full((nblk, block_size, dims.entry), 0x7F, dtype=torch.uint8, device=device)
            self.scales = torch.full((nblk, block_size, 2), fill, dtype=torch.float32, device=device)
        else:
            self.pool = torch.full((nblk, block_size, dims.entry), fill, dtype=torch_dtype(dims), device=device)
            self.scales = None
        self.table_np = table
        self.block_table = torch.from_numpy(table).to(device)
        self.ccache = make_cache(self.pool, self.block_table, self.scales)

    def clone(self) -> "PagedPool":
        c = PagedPool.__new__(PagedPool)
        c.dims, c.block_size, c.table_np, c.fp8 = self.dims, self.block_size, self.table_np, self.fp8
        c.pool = self.pool.clone()
        c.scales = None if self.scales is None else self.scales.clone()
        c.block_table = self.block_table.clone()
        c.ccache = make_cache(c.pool, c.block_table, c.scales)
        return c

    def _slots(self, b: int, n: int):
        pos = np.arange(n)
        blk = torch.from_numpy(self.table_np[b, pos // self.block_size].astype(np.int64)).to(self.pool.device)
        off = torch.from_numpy((pos % self.block_size).astype(np.int64)).to(self.pool.device)
        return blk, off

    def read_codes(self, b: int, n: int):
        """fp8 pool: codes [n, entry] uint8 and scales [n, 2] fp32 of positions 0..n-1 of sequence b."""
        blk, off = self._slots(b, n)
        return self.pool[blk, off].cpu().numpy(), self.scales[blk, off].cpu().numpy()

    def write_codes(self, b: int, codes: torch.Tensor, scales: torch.Tensor) -> None:
        """fp8 pool: stores device codes [n, entry] and scales [n, 2] at positions 0..n-1 of sequence b."""
        blk, off = self._slots(b, codes.shape[0])
        self.pool[blk, off] = codes
        self.scales[blk, off] = scales

    def read_entries(self, b: int, n: int) -> np.ndarray:
        """Entries of positions 0..n-1 of sequence b, as fp32 numpy [n, d_c + d_hr]."""
        if n == 0:
            return np.zeros((0, self.dims.entry), np.float32)
        pos = np.arange(n)
        blk = torch.from_numpy(self.table_np[b, pos // self.block_size].astype(np.int64)).to(self.pool.device)
        off = torch.from_numpy((pos % self.block_size).astype(np.int64)).to(self.pool.device)
        return self.pool[blk, off].float().cpu().numpy()

    def write_entries(self, b: int, entries: torch.Tensor) -> None:
        """Stores device entries [n, d_c + d_hr] at positions 0..n-1 of sequence b (a test input
        path that bypasses the cache writer)."""
        n = entries.shape[0]
        pos = np.arange(n)
        blk = torch.from_numpy(self.table_np[b, pos // self.block_size].astype(np.int64)).to(self.pool.device)
        off = torch.from_numpy((pos % self.block_size).astype(np.int64)).to(self.pool.device)
        self.pool[blk, off] = entries.to(self.pool.dtype)


def ws_tensor(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def build_context(layer: DeviceLayer, pool: PagedPool, lens, recipe: str, chunk: int = 8192, threads: int = 0):
    """Writes positions 0..lens[b]-1 of every sequence b into the pool through mla_cache_append,
    from the seeded hidden-state history of that sequence."""
    dims = layer.dims
    lens = [int(x) for x in lens]
    ws = ws_tensor(workspace_size(layer.cdims, OP_CACHE_APPEND, max_tokens=chunk))
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max(1, threads or 8)) as ex:
        futs = [ex.submit(S.hidden_history, dims, b, lens[b], recipe) for b in range(len(lens))]
        for b, f in enumerate(futs):
            h = f.result()
            for s0 in range(0, lens[b], chunk):
                n = min(chunk, lens[b] - s0)
                hd = to_device(h[s0:s0 + n], dims, layer.device)
                seq = torch.full((n,), b, dtype=torch.int32, device=layer.device)
                pos = torch.arange(s0, s0 + n, dtype=torch.int32, device=layer.device)
                cache_append(layer.cdims, layer.cweights, pool.ccache, hd, seq, pos, ws)
            futs[b] = None
    torch.cuda.synchronize()


def decode_workspace(layer: DeviceLayer, batch: int, max_ctx_len: int, num_splits: int = 0) -> torch.Tensor:
    return ws_tensor(workspace_size(layer.cdims, OP_DECODE, batch=batch, max_ctx_len=max_ctx_len,
                                    num_splits=num_splits), layer.device)


def prefill_workspace(layer: DeviceLayer, batch: int, T: int) -> torch.Tensor:
    return ws_tensor(workspace_size(layer.cdims, OP_PREFILL, batch=batch, max_tokens=T), layer.device)


def chunk_workspace(layer: DeviceLayer, batch: int, T: int, max_start: int) -> torch.Tensor:
    return ws_tensor(workspace_size(layer.cdims, OP_PREFILL_CHUNK, batch=batch, max_tokens=T, max_ctx_len=max_start),
                     layer.device)
