"""Benchmark of the MLA decode hot path on one MI355X.

A step is one full `mla_decode` call over the whole batch: query projections and RoPE, the
cache writer for the new tokens, the W_UK absorption, split-KV latent attention and its
reduction, W_UV and W_O.  Default workload: DeepSeek-V2 dims, batch 64, 8192 cached tokens per
sequence in a paged bf16 latent cache (block 64), decode at position 8192.

Inputs are seeded and synthetic and already resident in HBM when the timed region starts.
Steps rotate over independent replicas of the weights and the cache so that no step is served
from the previous step's cache lines.  The dominant kernel (decode attention) is timed in a
second loop of the attention-core entry point with HIP events on the stream it runs on.  The
fp64 oracle is timed on the host cores on a bounded sample as a CPU baseline.

Prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3
METRIC = "MLA decode tokens/s + achieved GB/s & %roofline, DeepSeek-V2 shape, 1 GPU"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    # After an idle spell the first few decode steps run fast and the next ~20 run 10-25% slower
    # (the GPU's power management reacting to the burst) before the rate settles.  The steps are
    # therefore run untimed for this long before the warm-up, so that the timed ones see the
    # steady state whatever --warmup is; 0 disables it.
    ap.add_argument("--settle-ms", type=float, default=300.0)
    ap.add_argument("--workload", default="v2_decode_b64_ctx8192")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--replicas", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["attn", "copy", "stream"], default=None,
                    help="profiling runs: only the attention core of the workload, only a plain device copy "
                         "of 1 GiB (the reference for HBM byte counters), or only the HBM streaming-ceiling "
                         "probe (every variant); prints one line")
    return ap.parse_args()


def copy_only(args):
    """A plain 1 GiB device-to-device copy, --warmup + --steps times (counter reference)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    print(json.dumps({"only": "copy", "bytes_read": n, "bytes_written": n, "ms": round(ms, 5),
                      "GBps": round(2 * n / (ms / 1e3) / 1e9, 1)}))


STREAM_BYTES = 2 << 30  # read passes over 2 GiB: eight times the 256 MB last-level cache
STREAM_VARIANTS = {0: "regs x2", 1: "regs x4", 2: "regs x8", 3: "regs x16", 4: "lds ring 4", 5: "lds ring 8",
                   6: "lds ring 16", 7: "operand-shaped x8", 8: "operand-shaped x16"}


def stream_ceiling(variants=None, blocks=(256, 512, 1024, 2048), reps=5):
    """Measured HBM read ceiling: the best GB/s over the probe's read-only passes (libmla_probe.so)
    on a 2 GiB buffer, each configuration timed over `reps` passes after one untimed pass."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "mla_latent_kv_27_amd", "lib", "libmla_probe.so"))
    lib.mla_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_void_p, ctypes.c_void_p]
    lib.mla_probe_stream_read.restype = ctypes.c_int
    buf = torch.empty(STREAM_BYTES, dtype=torch.uint8, device="cuda").fill_(3)
    sink = torch.empty(max(blocks), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    res = {}
    for v in (variants if variants is not None else STREAM_VARIANTS):
        for nb in blocks:
            def run():
                rc = lib.mla_probe_stream_read(buf.data_ptr(), STREAM_BYTES, v, nb, sink.data_ptr(), stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"stream probe variant {v} blocks {nb}: status {rc}")
            run()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                run()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            res[f"{STREAM_VARIANTS[v]}, {nb} blocks"] = round(STREAM_BYTES / (ms / 1e3) / 1e9, 1)
    del buf
    best = max(res, key=res.get)
    return {"GBps": res[best], "best": best, "bytes_per_pass": STREAM_BYTES, "all": res}


def entry_bytes(dims, cache="native"):
    """Bytes of one cached entry: bf16/fp32 values, or e4m3 codes plus two fp32 scales."""
    if cache == "fp8":
        return dims.entry + 8
    return dims.entry * (2 if dims.dtype == "bf16" else 4)


def decode_bytes(dims, lens, B, cache="native"):
    """Algorithmic HBM bytes of one decode step: each cached entry once, each weight once, h in,
    u out, the new entries written."""
    es = 2 if dims.dtype == "bf16" else 4
    eb = entry_bytes(dims, cache)
    cache_b = sum(int(L) + 1 for L in lens) * eb
    weights = dims.param_count() * es
    io = B * 2 * dims.d_model * es + B * eb
    return cache_b, weights, io


def decode_flops(dims, lens, B):
    attn = sum(int(L) + 1 for L in lens) * 2 * dims.n_h * (dims.entry + dims.d_c)
    proj = 2 * B * dims.param_count()
    return attn, proj


def attn_core_bytes(dims, lens, B, cache="native"):
    """Algorithmic bytes of the attention core: cached entries, the absorbed queries and o_hat."""
    es = 2 if dims.dtype == "bf16" else 4
    return sum(int(L) + 1 for L in lens) * entry_bytes(dims, cache) + B * dims.n_h * (dims.entry + dims.d_c) * es


def counters_for(kernel_file, workload):
    """HBM traffic per dispatch from a committed rocprofv3 counter summary, if it was taken on the
    current source of the kernel; else None."""
    path = os.path.join(ROOT, "profiles", f"decode_attn_{workload}.counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    # the kernel's source and the shared header it includes (copy helpers, waits)
    csrc = os.path.join(ROOT, "mla_latent_kv_27_amd", "csrc")
    src = open(os.path.join(csrc, kernel_file), "rb").read() + open(os.path.join(csrc, "common.h"), "rb").read()
    if kv.get("kernel_source_sha256") != hashlib.sha256(src).hexdigest():
        return None
    try:
        return float(kv["hbm_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(dims, W_np, lens, recipe, budget_s):
    """The fp64 oracle, un-absorbed, on whole sequences of the same workload until the budget is
    spent (at least one sequence); tokens/s = sequences decoded per second."""
    import numpy as np
    import mla_synth as S
    import oracle.mla_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    h = S.hidden_step(dims, len(lens), recipe)
    done, spent = 0, 0.0
    while done < len(lens) and (done == 0 or spent < budget_s):
        b = done
        cache = O.latent_entries(W_np, dims, S.hidden_history(dims, b, int(lens[b]), recipe), np.arange(int(lens[b])))
        t0 = time.perf_counter()
        O.mla_decode(W_np, dims, h[b:b + 1], [cache])
        spent += time.perf_counter() - t0
        done += 1
    return {"value": done / spent, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {len(lens)} sequences of the same decode step (each over {int(lens[0]) + 1} "
                      f"cached tokens), un-absorbed fp64 numpy, {spent:.1f} s; cache entries precomputed untimed"}


def prefill_flops(dims, T, B):
    """Causal attention over key <= query, un-absorbed (d_qk = d_h + d_hr, d_v = d_h), plus every
    weight applied once per token."""
    attn = B * 2 * dims.n_h * (dims.d_h + dims.d_hr + dims.d_h) * T * (T + 1) // 2
    return attn, 2 * B * T * dims.param_count()


def prefill_bench(args, w):
    """A step is one mla_prefill of the workload's sequences (projections, cache writer, causal
    attention, W_O); MFMA-bound, reported against the dense bf16 peak."""
    import numpy as np
    import torch
    import mla_synth as S
    import mla_latent_kv_27_amd as M
    from mla_latent_kv_27_amd import workload as WL

    dims, B, T = w.dims, w.batch, w.tokens
    torch.cuda.set_device(0)
    W_np = S.make_weights(dims, std=w.weight_std)
    layer = WL.DeviceLayer(dims, W_np)
    pool = WL.PagedPool(dims, [T] * B, block_size=w.block_size)
    h_np = np.stack(S.hidden_histories(dims, [T] * B, w.hidden))
    h = WL.to_device(h_np.reshape(B, T, dims.d_model), dims)
    u = torch.empty((B, T, dims.d_model), dtype=WL.torch_dtype(dims), device="cuda")
    ws = WL.prefill_workspace(layer, B, T)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        M.prefill(layer.cdims, layer.cweights, pool.ccache, h, u, ws, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        M.prefill(layer.cdims, layer.cweights, pool.ccache, h, u, ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    attn_f, proj_f = prefill_flops(dims, T, B)
    tflops = (attn_f + proj_f) / (ms / 1e3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        import oracle.mla_oracle as O
        n = min(T, 256)
        t0 = time.perf_counter()
        O.mla_prefill(W_np, dims, h_np[0, :n])
        dt = time.perf_counter() - t0
        cpu = {"value": n / dt, "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"the first {n} tokens of sequence 0 (causal, un-absorbed fp64 numpy), {dt:.1f} s; "
                         f"longer prefixes cost more per token"}
    rec = {"metric": "MLA prefill tokens/s (causal, writes the latent cache), DeepSeek-V2 shape, 1 GPU",
           "value": round(B * T / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": dims.dtype,
           "data": "synthetic (seeded weights N(0,0.02), RMS-normalised N(0,1) hidden states, random page order)",
           "config": {"workload": w.name, "batch": B, "tokens": T, "d_model": dims.d_model, "n_h": dims.n_h,
                      "d_h": dims.d_h, "d_c": dims.d_c, "d_cq": dims.d_cq, "d_hr": dims.d_hr},
           "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "traffic": None,
                        "kernel": "whole mla_prefill call (projections, cache writer, causal attention, W_O)",
                        "attention_flops": attn_f, "projection_flops": proj_f},
           "cpu_baseline": cpu}
    print(json.dumps(rec))


def chunk_flops(dims, P, T, B):
    """Chunked prefill of T tokens after P cached ones: causal attention of the chunk over P + i + 1
    keys (d_qk = d_h + d_hr, d_v = d_h), the per-head keys and values rebuilt from all P + T
    latents, and the other weights applied once per new token."""
    attn = B * 2 * dims.n_h * (dims.d_h + dims.d_hr + dims.d_h) * (T * P + T * (T + 1) // 2)
    rebuild = B * 2 * 2 * (P + T) * dims.d_c * dims.n_h * dims.d_h
    per_token = dims.param_count() - 2 * dims.n_h * dims.d_h * dims.d_c  # all but W_UK, W_UV
    return attn, rebuild + 2 * B * T * per_token


def chunk_bench(args, w):
    """A step is one mla_prefill_chunk: the next w.tokens tokens of each sequence after w.ctx
    cached ones (the same chunk slots are rewritten every step); MFMA-bound."""
    import numpy as np
    import torch
    import mla_synth as S
    import mla_latent_kv_27_amd as M
    from mla_latent_kv_27_amd import workload as WL

    dims, B, T, P = w.dims, w.batch, w.tokens, w.ctx
    torch.cuda.set_device(0)
    W_np = S.make_weights(dims, std=w.weight_std)
    layer = WL.DeviceLayer(dims, W_np)
    pool = WL.PagedPool(dims, [P + T] * B, block_size=w.block_size)
    WL.build_context(layer, pool, [P] * B, w.hidden)
    h_np = np.stack([S.hidden_history(dims, b, P + T, w.hidden)[P:] for b in range(B)])
    h = WL.to_device(h_np, dims)
    u = torch.empty((B, T, dims.d_model), dtype=WL.torch_dtype(dims), device="cuda")
    start = torch.full((B,), P, dtype=torch.int32, device="cuda")
    ws = WL.chunk_workspace(layer, B, T, P)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        M.prefill_chunk(layer.cdims, layer.cweights, pool.ccache, h, start, P, u, ws, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        M.prefill_chunk(layer.cdims, layer.cweights, pool.ccache, h, start, P, u, ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    attn_f, other_f = chunk_flops(dims, P, T, B)
    tflops = (attn_f + other_f) / (ms / 1e3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        import oracle.mla_oracle as O
        n = min(T, 32)
        prefix = O.latent_entries(W_np, dims, S.hidden_history(dims, 0, P, w.hidden), np.arange(P))
        t0 = time.perf_counter()
        O.mla_prefill(W_np, dims, h_np[0, :n], start_pos=P, prefix_cache=prefix)
        dt = time.perf_counter() - t0
        cpu = {"value": n / dt, "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"the first {n} chunk tokens of sequence 0 after its {P} cached ones (un-absorbed fp64 "
                         f"numpy), {dt:.1f} s; prefix entries precomputed untimed"}
    rec = {"metric": "MLA chunked prefill tokens/s (chunk after a cached prefix), DeepSeek-V2 shape, 1 GPU",
           "value": round(B * T / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": dims.dtype,
           "data": "synthetic (seeded weights N(0,0.02), RMS-normalised N(0,1) hidden states, random page order)",
           "config": {"workload": w.name, "batch": B, "prefix_tokens": P, "chunk_tokens": T, "d_model": dims.d_model,
                      "n_h": dims.n_h, "d_h": dims.d_h, "d_c": dims.d_c, "d_cq": dims.d_cq, "d_hr": dims.d_hr},
           "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "traffic": None,
                        "kernel": "whole mla_prefill_chunk call (projections, writer, prefix gather, key/value "
                                  "rebuild, causal attention, W_O)",
                        "attention_flops": attn_f, "other_flops": other_f},
           "cpu_baseline": cpu}
    print(json.dumps(rec))


def main():
    args = parse()
    if args.only == "copy":
        copy_only(args)
        return
    if args.only == "stream":
        import torch
        torch.cuda.set_device(0)
        print(json.dumps({"only": "stream", **stream_ceiling()}))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported: the library has no "
              f"multi-GPU path (decode shards by batch, one independent process per GPU)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import mla_synth as S
    import mla_latent_kv_27_amd as M
    from mla_latent_kv_27_amd import workload as WL

    w = S.WORKLOADS[args.workload]
    if w.kind == "prefill":
        prefill_bench(args, w)
        return
    if w.kind == "chunk":
        chunk_bench(args, w)
        return
    dims = w.dims
    torch.cuda.set_device(0)
    lens = S.context_lengths(w)
    B = w.batch
    max_ctx = int(max(lens))
    W_np = S.make_weights(dims, std=w.weight_std)
    fp8 = w.cache == "fp8"
    layer = WL.DeviceLayer(dims, W_np, cache_dtype="fp8" if fp8 else 0)
    pool = WL.PagedPool(dims, [int(L) + 1 for L in lens], block_size=w.block_size, fp8=fp8)
    t0 = time.perf_counter()
    WL.build_context(layer, pool, lens, w.hidden)
    setup_s = time.perf_counter() - t0
    h = WL.to_device(S.hidden_step(dims, B, w.hidden), dims)
    ctx = torch.tensor(np.asarray(lens, dtype=np.int32), device="cuda")
    # 0: the library's automatic choice (fixed partitions, or balanced units for small batches)
    splits = args.splits if args.splits > 0 else 0
    reps = [(layer, pool)] + [(layer.clone(), pool.clone()) for _ in range(max(0, args.replicas - 1))]
    outs = [torch.empty((B, dims.d_model), dtype=WL.torch_dtype(dims), device="cuda") for _ in reps]
    wss = [WL.decode_workspace(layer, B, max_ctx, splits) for _ in reps]
    stream = torch.cuda.current_stream()
    q = WL.to_device(S.to_dtype((np.random.default_rng(9).standard_normal((B, dims.n_h, dims.entry)) * 0.05)
                                .astype(np.float32), dims.dtype), dims)
    kv = ctx + 1
    ohat = torch.empty((B, dims.n_h, dims.d_c), dtype=WL.torch_dtype(dims), device="cuda")

    def auto_label(n):  # the library's rule: balanced units below 16 (sequence, head-group) units
        if B * ((dims.n_h + 127) // 128) < 16:
            return f"auto (balanced units, up to {min(128, 2 * n)} partitions per sequence)"
        return f"auto ({n} partitions per sequence)"

    # the attention kernel alone, as the step runs it: the KV partitions of the step's automatic
    # choice (fixed partitions; a small batch's step balances them over its lengths instead), left
    # as partials (the step combines them inside the W_UV kernel)
    att_splits = splits if splits > 0 else M.auto_splits(layer.cdims, B, max_ctx)
    pm = torch.empty((B, att_splits, dims.n_h), dtype=torch.float32, device="cuda")
    pl = torch.empty_like(pm)
    po = torch.empty((B, att_splits, dims.n_h, dims.d_c), dtype=torch.bfloat16, device="cuda")

    def attn(i):
        M.decode_attention_partials(layer.cdims, reps[i % len(reps)][1].ccache, q, kv, max_ctx + 1, att_splits,
                                    pm, pl, po, stream=stream)

    def settle(fn):
        """Untimed steps for --settle-ms of wall time; returns how many ran."""
        n, t_end = 0, time.perf_counter() + args.settle_ms / 1e3
        while time.perf_counter() < t_end:
            for _ in range(32):
                fn(n)
                n += 1
            torch.cuda.synchronize()
        return n

    def timed(fn, per_step=None):
        """Mean ms over exactly --steps calls after --warmup untimed ones (events on the stream the
        kernels run on, synchronised on both sides); per_step (a list) receives each call's ms."""
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        ev[0].record(stream)
        for i in range(args.steps):
            fn(i)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        if per_step is not None:
            per_step.extend(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
        return ev[0].elapsed_time(ev[-1]) / args.steps

    if args.only == "attn":
        settle(attn)
        attn_ms = timed(attn)
        print(json.dumps({"only": "attn", "workload": w.name, "num_splits": splits, "ms": round(attn_ms, 5),
                          "algorithmic_bytes": attn_core_bytes(dims, lens, B, w.cache)}))
        return

    def step(i):
        ly, pl = reps[i % len(reps)]
        M.decode(ly.cdims, ly.cweights, pl.ccache, h, ctx, max_ctx, outs[i % len(reps)], wss[i % len(reps)],
                 num_splits=splits, stream=stream)

    settled = settle(step)
    per_step = []
    ms = timed(step, per_step)
    value = B / (ms / 1e3)
    # dominant kernel: the latent attention core, timed on the same stream
    settle(attn)
    attn_ms = timed(attn)
    ceiling = stream_ceiling(variants=(2, 3), blocks=(256,), reps=5)
    core_bytes = attn_core_bytes(dims, lens, B, w.cache)
    achieved = core_bytes / (attn_ms / 1e3) / 1e9
    traffic = counters_for("decode_attn.hip", args.workload)

    cache_b, weight_b, io_b = decode_bytes(dims, lens, B, w.cache)
    step_bytes = cache_b + weight_b + io_b
    attn_f, proj_f = decode_flops(dims, lens, B)
    cpu = None
    if not args.no_cpu_baseline and not fp8:  # the oracle baseline is timed on the bf16 cache only
        cpu = cpu_baseline(dims, W_np, lens, w.hidden, args.cpu_seconds)

    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dims.dtype,
        "data": "synthetic (seeded weights N(0,0.02), RMS-normalised N(0,1) hidden states, random page order)",
        "config": {"workload": w.name, "batch": B, "ctx_tokens": [int(min(lens)), int(max(lens))],
                   "d_model": dims.d_model, "n_h": dims.n_h, "d_h": dims.d_h, "d_c": dims.d_c, "d_cq": dims.d_cq,
                   "d_hr": dims.d_hr, "block_size": w.block_size,
                   "num_splits": splits if splits > 0 else auto_label(M.auto_splits(layer.cdims, B, max_ctx)),
                   "replicas": len(reps),
                   "cache": "fp8_e4m3 (per-token scales)" if fp8 else dims.dtype,
                   "latent_rmsnorm": bool(dims.latent_norm),
                   "yarn_scale": float(dims.rope_scale) if dims.rope_scale > 1 else None},
        "settle_steps": settled,
        "step_ms_p10_p50_p90": [round(float(np.percentile(per_step, x)), 5) for x in (10, 50, 90)],
        "step_GBps": round(step_bytes / (ms / 1e3) / 1e9, 1),
        "step_hbm_frac": round(step_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
        "step_bytes": step_bytes,
        "step_TFLOPs": round((attn_f + proj_f) / (ms / 1e3) / 1e12, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": f"decode_attn_tiled_kernel{' over the fp8 cache' if fp8 else ''} "
                               f"(mla_decode_attention_partials, {att_splits} KV "
                               f"partitions per sequence, partials left for the W_UV kernel as in the step)",
                     "kernel_ms": round(attn_ms, 5), "algorithmic_bytes": core_bytes,
                     "measured_peak": ceiling["GBps"],
                     "frac_of_measured": round(achieved / ceiling["GBps"], 4),
                     "measured_peak_probe": f"best read-only pass over {STREAM_BYTES >> 30} GiB ({ceiling['best']})",
                     "mfma_TFLOPs": round(attn_f / (attn_ms / 1e3) / 1e12, 1),
                     "mfma_frac": round(attn_f / (attn_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
