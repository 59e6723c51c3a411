"""Throughput of the chunked H2O attention step on one MI355X.

One step = one whole synthetic sequence of the named workload through the C
ABI: cache reset, the prefill chunk (N_C tokens), then every chunk step of
length S up to the total length.  Inputs are generated on the host from the
seeded generators and uploaded before timing, so they are resident in HBM
when the timed region starts.

Reported (one JSON line): algorithmic TFLOP/s of the attention (4 d flops per
visible (query, key) pair per query head; the score pass's recompute is not
counted), tokens/s, the roofline of the dominant kernel (attention forward,
bf16 MFMA) from HIP events recorded by the library on the launch stream, and
the fp64 CPU oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0


def algorithmic_flops(w, with_prefill=True):
    """Per-launch attention flops of a whole sequence: list of (kind, flops)."""
    d, B, Hq, M = w.head_dim, w.batch, w.n_q_heads, w.cache_slots
    out = []
    T = 0
    for c in range(w.n_chunks):
        _, n = w.chunk_bounds(c)
        mv = min(T, M)
        visible = n * mv + n * (n + 1) // 2
        if c > 0 or with_prefill:
            out.append(("prefill" if c == 0 else "chunk", 4.0 * B * Hq * d * visible))
        T += n
    return out


def oracle_sample(w, seed, budget_s=20.0):
    """Times the fp64 oracle on the first chunks of the workload (prefill plus
    as many chunk steps as fit in about `budget_s`), all heads."""
    from oracle import h2o_oracle as orc
    from kv_cache_eviction_amd import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    hh = wl.heavy_hitters(w, seed)
    flops = algorithmic_flops(w)
    K, V, sig, pos = orc.empty_state(w.batch, w.n_kv_heads, w.cache_slots, w.head_dim)
    done_flops = 0.0
    tokens = 0
    elapsed = 0.0
    T = 0
    c = 0
    while c < w.n_chunks and elapsed < budget_s:
        q, k, v = (wl.stored_to_f64(x) for x in wl.chunk_inputs(w, seed, c, hh=hh))
        t0 = time.perf_counter()
        st = orc.chunk_step(K, V, sig, pos, T, q, k, v, w.recent_window)
        elapsed += time.perf_counter() - t0
        K, V, sig, pos, T = st["K"], st["V"], st["sigma"], st["pos"], st["T"]
        done_flops += flops[c][1]
        tokens += w.batch * q.shape[2]
        c += 1
    return dict(value=done_flops / elapsed / 1e12, unit="TFLOP/s", cores=int(threads), kind="oracle",
                sample=f"prefill + {c - 1} chunk steps of {w.name} (all heads), {elapsed:.1f} s",
                tokens_per_s=tokens / elapsed)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_64k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the H2O step shards by batch or KV head with no "
              f"exchange); --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    from kv_cache_eviction_amd import workloads as wl
    from kv_cache_eviction_amd import h2o

    w = wl.workload(args.workload)
    cfg = h2o.H2OConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.cache_slots,
                        w.recent_window, w.chunk, w.prefill, w.dtype)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hh = wl.heavy_hitters(w, args.seed)

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    chunks = []
    for c in range(w.n_chunks):
        q, k, v = wl.chunk_inputs(w, args.seed, c, hh=hh)
        chunks.append((up(q), up(k), up(v)))
    outs = [torch.empty_like(q) for q, _, _ in chunks]
    lses = [torch.empty(q.shape[:3], dtype=torch.float32, device=dev) for q, _, _ in chunks]
    B, Hkv, M, d = w.batch, w.n_kv_heads, w.cache_slots, w.head_dim
    k_cache = torch.zeros((B, Hkv, M, d), dtype=cfg.torch_dtype, device=dev)
    v_cache = torch.zeros_like(k_cache)
    scores = torch.empty((B, Hkv, M), dtype=torch.float32, device=dev)
    positions = torch.empty((B, Hkv, M), dtype=torch.int32, device=dev)
    workspace = torch.empty(h2o.h2o_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    timing_handles = []

    def one_pass(timing):
        handle = h2o.h2o_cache_init(cfg, k_cache, v_cache, scores, positions, workspace, stream=stream)
        if timing:
            h2o.h2o_set_timing(handle, timing)
        q, k, v = chunks[0]
        h2o.h2o_prefill(handle, cfg, q, k, v, outs[0], lses[0], stream)
        for c in range(1, w.n_chunks):
            q, k, v = chunks[c]
            h2o.h2o_chunk_step(handle, cfg, q, k, v, outs[c], lses[c], stream=stream)
        return handle

    for _ in range(args.warmup):
        h2o.h2o_cache_destroy(one_pass(None))
    torch.cuda.synchronize()
    # timed region: only the attention kernel is bracketed with library events
    # (two extra stream records per step); each pass is bracketed too, for the
    # per-step median
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        marks[i][0].record(stream)
        timing_handles.append(one_pass(["attn_fwd"]))
        marks[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    pass_ms = sorted(a.elapsed_time(b) for a, b in marks)
    attn_ms, attn_n = 0.0, 0
    for hd in timing_handles:
        ms, cnt = h2o.h2o_get_timing(hd, "attn_fwd")
        attn_ms += ms
        attn_n += cnt
        h2o.h2o_cache_destroy(hd)

    # per-kernel breakdown: one more pass with every kernel bracketed (outside
    # the timed region; its event records slow that pass slightly)
    hd = one_pass(True)
    torch.cuda.synchronize()
    step_ms = {}
    for name in ("attn_fwd", "score", "select", "scatter", "reset"):
        ms, cnt = h2o.h2o_get_timing(hd, name)
        step_ms[name] = ms
    h2o.h2o_cache_destroy(hd)

    fl = algorithmic_flops(w)
    flops_per_step = sum(f for _, f in fl)
    tflops = flops_per_step / (ms_per_step * 1e-3) / 1e12
    tokens_per_s = w.batch * w.total_len / (ms_per_step * 1e-3)
    attn_avg_ms = attn_ms / max(attn_n, 1)
    achieved = flops_per_step * args.steps / (attn_ms * 1e-3) / 1e12 if attn_ms > 0 else None
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    chunk_flops = [f for k, f in fl if k == "chunk"]

    cpu = None
    if not args.no_cpu_baseline:
        cpu = oracle_sample(w, args.seed, args.cpu_budget)

    rec = {
        "metric": "H2O chunk-step TFLOP/s + tokens/s at 64k ctx, 8B-GQA shape; % of roofline",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": round(pass_ms[len(pass_ms) // 2], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded generators, no dataset or weights)",
        "config": {
            "workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
            "head_dim": w.head_dim, "prefill": w.prefill, "chunk": w.chunk, "total_len": w.total_len,
            "cache_slots": w.cache_slots, "recent_window": w.recent_window,
            "step": "cache reset + prefill + %d chunk steps" % w.n_steps,
        },
        "tokens_per_s": round(tokens_per_s, 1),
        "roofline": {
            "bound": "mfma", "kernel": "attn_fwd_bf16_kernel" if w.dtype == "bf16" else "attn_fwd_f32_kernel",
            "achieved": None if achieved is None else round(achieved, 2), "peak": peak,
            "unit": "TFLOP/s", "frac": None if achieved is None else round(achieved / peak, 4),
            "traffic": None, "avg_launch_us": round(attn_avg_ms * 1e3, 3),
            "chunk_step_flops": chunk_flops[0] if chunk_flops else None,
        },
        "kernel_ms_per_step": {k: round(v, 4) for k, v in step_ms.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
