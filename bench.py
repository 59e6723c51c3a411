"""Throughput of the chunked H2O attention step on one MI355X.

One step = one whole synthetic sequence of the named workload through the C
ABI: cache reset, the prefill chunk (N_C tokens), then every chunk step of
length S up to the total length (with the frozen-eviction backward after
each chunk step for the workload that trains through the lattice).  Inputs
are generated on the host from the seeded generators and uploaded before
timing, so they are resident in HBM when the timed region starts.

Reported (one JSON line): algorithmic TFLOP/s of the attention (4 d flops per
visible (query, key) pair per query head forward, 10 d backward; the score
pass's recompute is not counted), tokens/s, the roofline of the dominant
kernel (attention forward, or attention and masses in one kernel for short
chunks: bf16 MFMA, or HBM for the decode workload) from HIP events recorded
by the library on the launch stream around the prefill's launch and every
--event-stride-th chunk step's launch of the timed passes (a pair of event
records costs ~5 us of GPU time, so bracketing every launch would slow the
timed job itself), and the fp64 CPU oracle timed on a bounded sample of the
same workload.

With --recurrence (workloads with a backward): one step = the forward over
the whole row with every chunk step's buffer delta recorded, then the
backward walk through the buffer (h2o_recurrence_backward_step, last chunk
first, the prefill last), which gives every chunk's q/k/v their total
gradients.

With --policy recent | sink_recent (--n-sink N): the same step under a
position eviction policy (no score pass; the oldest unprotected tokens go).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--recurrence]
                       [--policy h2o|recent|sink_recent] [--n-sink N] [--no-cpu-baseline]
                       [--event-stride K]
       python bench.py --copy-probe MB    (plain copy of known size, for
                                           scaling the HBM byte counters)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0

# workloads whose metric is bytes (HBM-bound); their prefill only fills the
# cache and is not timed
HBM_BOUND = {"decode_b32"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")
# the dominant kernels' sources: each file and the device helpers it inlines
ATTN_SOURCES = [os.path.join(ROOT, "kv_cache_eviction_amd", "csrc", f) for f in ("attn_fwd.hip", "h2o_device.h")]
FUSED_SOURCES = [os.path.join(ROOT, "kv_cache_eviction_amd", "csrc", f) for f in ("decode.hip", "h2o_device.h")]


def takes_fused_kernel(w, policy):
    """True when the chunk steps run the attention and the column masses in
    one kernel: the library's rule for an H2O step (bf16, d 64 or 128, at most
    512 query rows per KV group, at most 72 blocks of 32 keys per head once the
    cache is full: ceil(M / 32) + ceil(S / 32))."""
    return (w.dtype == "bf16" and policy == "h2o" and w.head_dim in (64, 128) and w.group * w.chunk <= 512
            and (w.cache_slots + 31) // 32 + (w.chunk + 31) // 32 <= 72)


def visible_pairs(w, c, T):
    """Visible (query, key) pairs per query head of chunk c after T tokens."""
    _, n = w.chunk_bounds(c)
    mv = min(T, w.cache_slots)
    return n * mv + n * (n + 1) // 2


def algorithmic_flops(w, backward=False, prefill_backward=False):
    """Attention flops of a whole sequence, per launch: list of (kind, flops)."""
    d, B, Hq = w.head_dim, w.batch, w.n_q_heads
    out = []
    T = 0
    for c in range(w.n_chunks):
        v = visible_pairs(w, c, T)
        out.append(("prefill" if c == 0 else "chunk", 4.0 * B * Hq * d * v))
        if backward and (c > 0 or prefill_backward):
            out.append(("backward", 10.0 * B * Hq * d * v))
        T += w.chunk_bounds(c)[1]
    return out


def attn_bytes(w, c, T):
    """Algorithmic HBM bytes of one attention launch: Q in, O out, the valid
    cache rows of K and V once, the chunk's K and V, and lse."""
    _, n = w.chunk_bounds(c)
    e, B, Hq, Hkv, d = w.elem_bytes, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    mv = min(T, w.cache_slots)
    return e * (2 * B * Hq * n * d + 2 * B * Hkv * mv * d + 2 * B * Hkv * n * d) + 4 * B * Hq * n


def state_bytes(w, c):
    """Algorithmic HBM bytes of one step's H2O state beyond the attention:
    every slot's score read and written back (each gains its mass), every
    slot's position read once (filled or free, protected or not), and the
    chunk's K/V rows and positions written into their slots."""
    _, n = w.chunk_bounds(c)
    e, B, Hkv, d, M = w.elem_bytes, w.batch, w.n_kv_heads, w.head_dim, w.cache_slots
    return B * Hkv * (4 * M + 4 * M + 4 * M + 4 * n + 2 * n * d * e)


def source_digest(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel, workload, sources=ATTN_SOURCES):
    """HBM bytes per launch from the counter runs recorded in
    profiles/hbm_traffic.md, or None if absent or taken on another version of
    the kernel source."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    pat = re.compile(r"^\|\s*%s\s*\|\s*%s\s*\|\s*([0-9]+)\s*\|\s*([0-9a-f]+)\s*\|" % (
        re.escape(kernel), re.escape(workload)), re.M)
    m = pat.search(text)
    if not m or m.group(2) != source_digest(sources):
        return None
    return int(m.group(1))


def oracle_sample(w, seed, budget_s=20.0, policy="h2o", n_sink=0):
    """Times the fp64 oracle on the first chunks of the workload (prefill plus
    as many chunk steps as fit in about `budget_s`), all heads, forward."""
    from oracle import h2o_oracle as orc
    from kv_cache_eviction_amd import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    hh = wl.heavy_hitters(w, seed)
    flops = [f for k, f in algorithmic_flops(w)]
    K, V, sig, pos = orc.empty_state(w.batch, w.n_kv_heads, w.cache_slots, w.head_dim)
    done_flops = 0.0
    tokens = 0
    elapsed = 0.0
    T = 0
    c = 0
    while c < w.n_chunks and elapsed < budget_s:
        q, k, v = (wl.stored_to_f64(x) for x in wl.chunk_inputs(w, seed, c, hh=hh))
        t0 = time.perf_counter()
        st = orc.chunk_step(K, V, sig, pos, T, q, k, v, w.recent_window, policy=policy, n_sink=n_sink)
        elapsed += time.perf_counter() - t0
        K, V, sig, pos, T = st["K"], st["V"], st["sigma"], st["pos"], st["T"]
        done_flops += flops[c]
        tokens += w.batch * q.shape[2]
        c += 1
    return dict(value=done_flops / elapsed / 1e12, unit="TFLOP/s", cores=int(threads), kind="oracle",
                sample=f"prefill + {c - 1} chunk steps of {w.name} (all heads, forward), {elapsed:.1f} s",
                tokens_per_s=tokens / elapsed)


def plan_groups(batch, n_kv_heads, n):
    """How N independent caches divide the workload: ("batch", B / N) when the
    batch splits evenly and B > 1, ("heads", Hkv / N) when B == 1 and the KV
    heads split evenly, else None.  Every (sequence, KV head) pair runs its
    own eviction, so the groups share nothing."""
    if n < 1:
        return None
    if n == 1:
        return ("batch", batch)
    if batch > 1:
        return ("batch", batch // n) if batch % n == 0 else None
    return ("heads", n_kv_heads // n) if n_kv_heads % n == 0 else None


def copy_probe(mb):
    """A plain elementwise copy of a known size (reads mb MiB, writes mb MiB,
    three launches), so that HBM byte counters can be scaled to bytes."""
    import torch
    n = mb * 1024 * 1024 // 4
    a = torch.rand(n, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "launches": 3}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_64k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB")
    ap.add_argument("--recurrence", action="store_true",
                    help="forward over the row, then the backward walk through the buffer")
    ap.add_argument("--policy", default="h2o", choices=["h2o", "recent", "sink_recent"])
    ap.add_argument("--n-sink", type=int, default=4, help="sink tokens of the sink_recent policy")
    ap.add_argument("--event-stride", type=int, default=8, metavar="K",
                    help="in the timed passes, bracket every K-th chunk step's attention launch with events "
                         "(a pair of event records costs ~5 us of GPU time on the part)")
    ap.add_argument("--streams", type=int, default=1, metavar="N",
                    help="run the workload's independent (sequence, KV head) pairs as N caches on N streams: "
                         "the batch split N ways when B > 1, the KV heads when B == 1 (forward steps only)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the H2O step shards by batch or KV head with no "
              f"exchange); --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    import torch
    from kv_cache_eviction_amd import workloads as wl
    from kv_cache_eviction_amd import h2o

    w = wl.workload(args.workload)
    hbm = w.name in HBM_BOUND
    backward = w.backward
    rec = args.recurrence
    if rec and not backward:
        print(f"--recurrence needs a workload with a backward (not {w.name})", file=sys.stderr)
        sys.exit(2)
    n_sink = args.n_sink if args.policy == "sink_recent" else 0
    ns = args.streams
    split = None
    if ns > 1:
        if rec or backward:
            print("--streams applies to forward-only workloads", file=sys.stderr)
            sys.exit(2)
        split = plan_groups(w.batch, w.n_kv_heads, ns)
        if split is None:
            print(f"--streams {ns} divides neither the batch ({w.batch}) nor the KV heads ({w.n_kv_heads})",
                  file=sys.stderr)
            sys.exit(2)
    cfg = h2o.H2OConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.cache_slots,
                        w.recent_window, w.chunk, w.prefill, w.dtype, policy=args.policy, n_sink=n_sink)
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
    if rec:
        # every step's buffer delta (the prefill's: slots 0..n-1 of empty
        # rows), the walk's carried fp32 slot gradients and its outputs
        n0 = chunks[0][0].shape[2]
        deltas = [(torch.arange(n0, dtype=torch.int32, device=dev).expand(B, Hkv, n0).contiguous(),
                   torch.zeros_like(chunks[0][1]), torch.zeros_like(chunks[0][2]),
                   torch.full((B, Hkv, n0), -1, dtype=torch.int32, device=dev))]
        for c in range(1, w.n_chunks):
            _, k, v = chunks[c]
            deltas.append((torch.empty(k.shape[:3], dtype=torch.int32, device=dev), torch.empty_like(k),
                           torch.empty_like(v), torch.empty(k.shape[:3], dtype=torch.int32, device=dev)))
        d_outs = [up(wl.chunk_grad_out(w, args.seed, c)) for c in range(w.n_chunks)]
        acc_k = torch.zeros((B, Hkv, M, d), dtype=torch.float32, device=dev)
        acc_v = torch.zeros_like(acc_k)
        rgrads = {}
        for c in (0, 1):
            q, k, _ = chunks[c]
            rgrads[q.shape[2]] = (torch.empty_like(q), torch.empty(k.shape, dtype=torch.float32, device=dev),
                                  torch.empty(k.shape, dtype=torch.float32, device=dev))
        rws = torch.empty(h2o.h2o_recurrence_workspace_bytes(cfg, max(w.prefill, w.chunk)), dtype=torch.uint8,
                          device=dev)
    elif backward:
        # the backward needs the pre-step cache: copied before each step (part of the job)
        k_pre, v_pre, pos_pre = torch.empty_like(k_cache), torch.empty_like(v_cache), torch.empty_like(positions)
        d_outs = [up(wl.chunk_grad_out(w, args.seed, c)) if c > 0 else None for c in range(w.n_chunks)]
        grads = [torch.empty_like(chunks[1][0]), torch.empty_like(k_cache), torch.empty_like(v_cache),
                 torch.empty_like(chunks[1][1]), torch.empty_like(chunks[1][2])]
        bws = torch.empty(h2o.h2o_backward_workspace_bytes(cfg, w.chunk), dtype=torch.uint8, device=dev)
    bwd_marks = []

    def one_pass(timing, marks=None, bwd_timing=False):
        handle = h2o.h2o_cache_init(cfg, k_cache, v_cache, scores, positions, workspace, stream=stream)
        # the decode workload's timed launches are its chunk steps (the
        # prefill only fills the cache); the others time the prefill too
        if timing and not hbm:
            h2o.h2o_set_timing(handle, timing)
        q, k, v = chunks[0]
        h2o.h2o_prefill(handle, cfg, q, k, v, outs[0], lses[0], stream)
        if timing and hbm:
            h2o.h2o_set_timing(handle, timing)
        if marks is not None:
            marks[0].record(stream)
        for c in range(1, w.n_chunks):
            q, k, v = chunks[c]
            if marks is not None and timing and args.event_stride > 1:
                h2o.h2o_set_timing(handle, timing if c % args.event_stride == 0 else False)
            if rec:
                sl, ko, vo, po = deltas[c]
                h2o.h2o_chunk_step(handle, cfg, q, k, v, outs[c], lses[c], slots_out=sl, k_old=ko, v_old=vo,
                                   pos_old=po, stream=stream)
                continue
            if backward:
                k_pre.copy_(k_cache)
                v_pre.copy_(v_cache)
                pos_pre.copy_(positions)
            h2o.h2o_chunk_step(handle, cfg, q, k, v, outs[c], lses[c], stream=stream)
            if backward:
                if bwd_timing:
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                h2o.h2o_chunk_backward(cfg, q, k_pre, v_pre, pos_pre, k, v, outs[c], lses[c], d_outs[c],
                                       *grads, bws, stream)
                if bwd_timing:
                    e1.record(stream)
                    bwd_marks.append((e0, e1))
        if rec:
            # the walk: last chunk first; the cache ends as the pass found it
            acc_k.zero_()
            acc_v.zero_()
            for c in reversed(range(w.n_chunks)):
                q, k, v = chunks[c]
                sl, ko, vo, po = deltas[c]
                dq, gk, gv = rgrads[q.shape[2]]
                if bwd_timing:
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                h2o.h2o_recurrence_backward_step(cfg, k_cache, v_cache, positions, sl, ko, vo, po, q, k, v,
                                                 outs[c], lses[c], d_outs[c], acc_k, acc_v, dq, gk, gv, rws,
                                                 stream)
                if bwd_timing:
                    e1.record(stream)
                    bwd_marks.append((e0, e1))
        if marks is not None:
            marks[1].record(stream)
        return handle

    if split is not None:
        # N caches, one per group, each on its own stream (default priority);
        # each group's steps stay in order on its stream, the groups meet only
        # at the pass's start and end
        kind, per = split
        G = w.n_q_heads // w.n_kv_heads
        if kind == "batch":
            cfgs = [h2o.H2OConfig(per, w.n_q_heads, w.n_kv_heads, w.head_dim, w.cache_slots, w.recent_window,
                                  w.chunk, w.prefill, w.dtype, policy=args.policy, n_sink=n_sink)] * ns

            def gview(t, g, heads):
                return t[g * per:(g + 1) * per]
        else:
            cfgs = [h2o.H2OConfig(1, per * G, per, w.head_dim, w.cache_slots, w.recent_window,
                                  w.chunk, w.prefill, w.dtype, policy=args.policy, n_sink=n_sink)] * ns

            def gview(t, g, heads):
                h = per * G if heads == "q" else per
                return t[:, g * h:(g + 1) * h]
        gstate = []
        for g in range(ns):
            cg = cfgs[g]
            kc = torch.zeros((cg.batch, cg.n_kv_heads, M, d), dtype=cfg.torch_dtype, device=dev)
            gstate.append(dict(
                k_cache=kc, v_cache=torch.zeros_like(kc),
                scores=torch.empty((cg.batch, cg.n_kv_heads, M), dtype=torch.float32, device=dev),
                positions=torch.empty((cg.batch, cg.n_kv_heads, M), dtype=torch.int32, device=dev),
                workspace=torch.empty(h2o.h2o_workspace_bytes(cg), dtype=torch.uint8, device=dev),
                stream=torch.cuda.Stream(device=dev),
                chunks=[(gview(q, g, "q"), gview(k, g, "kv"), gview(v, g, "kv"), gview(outs[c], g, "q"),
                         gview(lses[c], g, "q")) for c, (q, k, v) in enumerate(chunks)]))

        def fork():
            ev = torch.cuda.Event()
            ev.record(stream)
            for gs in gstate:
                gs["stream"].wait_event(ev)

        def join():
            for gs in gstate:
                ev = torch.cuda.Event()
                ev.record(gs["stream"])
                stream.wait_event(ev)

        def one_pass(timing, marks=None, bwd_timing=False):
            fork()
            hds = []
            for g, gs in enumerate(gstate):
                hd = h2o.h2o_cache_init(cfgs[g], gs["k_cache"], gs["v_cache"], gs["scores"], gs["positions"],
                                        gs["workspace"], stream=gs["stream"])
                if timing and not hbm:
                    h2o.h2o_set_timing(hd, timing)
                q, k, v, o, l = gs["chunks"][0]
                h2o.h2o_prefill(hd, cfgs[g], q, k, v, o, l, gs["stream"])
                if timing and hbm:
                    h2o.h2o_set_timing(hd, timing)
                hds.append(hd)
            if marks is not None:
                join()
                marks[0].record(stream)
                fork()
            for c in range(1, w.n_chunks):
                for g, gs in enumerate(gstate):
                    if marks is not None and timing and args.event_stride > 1:
                        h2o.h2o_set_timing(hds[g], timing if c % args.event_stride == 0 else False)
                    q, k, v, o, l = gs["chunks"][c]
                    h2o.h2o_chunk_step(hds[g], cfgs[g], q, k, v, o, l, stream=gs["stream"])
            join()
            if marks is not None:
                marks[1].record(stream)
            return hds

    def handles_of(r):
        return r if isinstance(r, list) else [r]

    for _ in range(args.warmup):
        for hd in handles_of(one_pass(None)):
            h2o.h2o_cache_destroy(hd)
    torch.cuda.synchronize()
    # timed region: only the attention kernel is bracketed with library events
    # (two extra stream records per step); the chunk steps of each pass are
    # bracketed too
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    handles = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        handles.extend(handles_of(one_pass(["attn_fwd"], marks[i])))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    chunk_ms = sorted(a.elapsed_time(b) for a, b in marks)     # chunk steps of each pass
    attn_ms, attn_n = 0.0, 0
    for hd in handles:
        ms, cnt = h2o.h2o_get_timing(hd, "attn_fwd")
        attn_ms += ms
        attn_n += cnt
        h2o.h2o_cache_destroy(hd)

    # per-kernel breakdown: one more pass with every kernel bracketed (outside
    # the timed region; its event records slow that pass slightly)
    hds = handles_of(one_pass(True, bwd_timing=backward))
    torch.cuda.synchronize()
    step_ms = {}
    for name in ("attn_fwd", "score", "select", "scatter", "reset"):
        step_ms[name] = sum(h2o.h2o_get_timing(hd, name)[0] for hd in hds)
    for hd in hds:
        h2o.h2o_cache_destroy(hd)
    if backward:
        step_ms["backward"] = sum(a.elapsed_time(b) for a, b in bwd_marks)

    fl = algorithmic_flops(w, backward, prefill_backward=rec)
    attn_fl = [f for kind, f in fl if kind != "backward"]
    # the attention launches the timed passes bracketed: the prefill's (not
    # on the HBM-bound workload) and every event_stride-th chunk step's
    timed_c = ([] if hbm else [0]) + [c for c in range(1, w.n_chunks) if c % max(args.event_stride, 1) == 0]
    attn_avg_ms = attn_ms / max(attn_n, 1)
    if attn_n != len(timed_c) * args.steps * ns:
        print(f"bench.py: {attn_n} bracketed attention launches, expected {len(timed_c) * args.steps * ns}",
              file=sys.stderr)
        sys.exit(3)
    if hbm:
        # the prefill only fills the cache: time and count the chunk steps
        ms_per_step = sum(chunk_ms) / args.steps
        ms_median = chunk_ms[len(chunk_ms) // 2]
        tflops = sum(f for kind, f in fl if kind != "prefill") / (ms_per_step * 1e-3) / 1e12
        tokens = w.batch * (w.total_len - w.prefill)
        T, abytes = 0, []
        for c in range(w.n_chunks):
            abytes.append(attn_bytes(w, c, T))
            T += w.chunk_bounds(c)[1]
        per_launch = sum(abytes[c] for c in timed_c) / len(timed_c)    # the bracketed chunk steps'
        if takes_fused_kernel(w, args.policy):
            # the kernel also writes one fp32 mass per key of every KV head
            T, mbytes = 0, []
            for c in range(w.n_chunks):
                mbytes.append(4 * w.batch * w.n_kv_heads * (min(T, w.cache_slots) + w.chunk_bounds(c)[1]))
                T += w.chunk_bounds(c)[1]
            per_launch += sum(mbytes[c] for c in timed_c) / len(timed_c)
            kernel, scope, srcs = "decode_fused_kernel", "attention and column-mass kernel", FUSED_SOURCES
        else:
            kernel, scope, srcs = "attn_fwd_bf16_kernel", "attention kernel only", ATTN_SOURCES
        per_launch /= ns                   # each group's launch covers 1/N of the pairs
        achieved = per_launch / (attn_avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": kernel, "scope": scope,
                "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": recorded_traffic(kernel, w.name, srcs) if ns == 1 else None,
                "avg_launch_us": round(attn_avg_ms * 1e3, 3), "algorithmic_bytes_per_launch": round(per_launch),
                "bracketed_launches": f"every {args.event_stride}th chunk step's, {attn_n} in the timed passes",
                **({"concurrent_streams": ns} if ns > 1 else {})}
        metric = "H2O decode-step algorithmic HBM GB/s of the chunk steps (B32, S16, M2048)"
        unit = "GB/s"
        value = round(sum(abytes[1:]) / (ms_per_step * 1e-3) / 1e9, 1)
        # the same steps with the H2O state they read and write counted too
        step_bytes = sum(abytes[1:]) + sum(state_bytes(w, c) for c in range(1, w.n_chunks))
        with_state = {"value": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1), "unit": "GB/s",
                      "bytes_per_step": round(step_bytes / w.n_steps),
                      "frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                      "counts": "the attention's bytes plus every slot's score read and written, every "
                                "slot's position read, the chunk's K/V rows and positions written"}
    else:
        ms_per_step = wall * 1e3 / args.steps
        ms_median = None
        tflops = sum(f for _, f in fl) / (ms_per_step * 1e-3) / 1e12
        tokens = w.batch * w.total_len
        per_launch = sum(attn_fl[c] for c in timed_c) / len(timed_c) / ns
        achieved = per_launch / (attn_avg_ms * 1e-3) / 1e12
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
        if takes_fused_kernel(w, args.policy):
            kernel, scope, srcs = "decode_fused_kernel", "attention and column-mass kernel", FUSED_SOURCES
        else:
            kernel = "attn_fwd_bf16_kernel" if w.dtype == "bf16" else "attn_fwd_f32_kernel"
            scope, srcs = "attention kernel only", ATTN_SOURCES
        roof = {"bound": "mfma", "kernel": kernel,
                "scope": scope, "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": recorded_traffic(kernel, w.name, srcs) if ns == 1 else None,
                "avg_launch_us": round(attn_avg_ms * 1e3, 3), "algorithmic_flops_per_launch": round(per_launch),
                "bracketed_launches": f"the prefill's and every {args.event_stride}th chunk step's, "
                                      f"{attn_n} in the timed passes",
                **({"concurrent_streams": ns} if ns > 1 else {})}
        metric = "H2O chunk-step TFLOP/s + tokens/s at 64k ctx, 8B-GQA shape; % of roofline"
        if rec:
            metric = ("H2O row TFLOP/s + tokens/s at %dk ctx, G=%d d=%d: forward, then the backward walk "
                      "through the KV buffer; %% of roofline" % (w.total_len // 1024, w.group, w.head_dim))
        elif w.name != "llama8b_64k":
            metric = "H2O chunk-step TFLOP/s + tokens/s at %dk ctx, G=%d d=%d%s; %% of roofline" % (
                w.total_len // 1024, w.group, w.head_dim, ", with the backward" if backward else "")
        if args.policy != "h2o":
            metric = "%s-policy chunk-step TFLOP/s + tokens/s at %dk ctx, G=%d d=%d%s; %% of roofline" % (
                args.policy, w.total_len // 1024, w.group, w.head_dim,
                " (n_sink %d)" % n_sink if n_sink else "")
        unit = "TFLOP/s"
        value = round(tflops, 3)
    tokens_per_s = tokens / (ms_per_step * 1e-3)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = oracle_sample(w, args.seed, args.cpu_budget, args.policy, n_sink)

    rec = {
        "metric": metric,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_chunk_steps_median": round(ms_median if ms_median is not None else chunk_ms[len(chunk_ms) // 2], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded generators, no dataset or weights)",
        "config": {
            "workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
            "head_dim": w.head_dim, "prefill": w.prefill, "chunk": w.chunk, "total_len": w.total_len,
            "cache_slots": w.cache_slots, "recent_window": w.recent_window, "policy": args.policy,
            **({"n_sink": n_sink} if n_sink else {}),
            **({"streams": ns, "groups": "%d caches of %s" % (ns, "%d sequences" % split[1] if split[0] == "batch"
                                                              else "%d KV heads" % split[1])} if ns > 1 else {}),
            "step": ("cache reset + prefill + %d chunk steps recording their buffer deltas, then the "
                     "backward walk over all %d steps (last first)" % (w.n_steps, w.n_chunks)) if rec else
                    "%s + %d chunk steps%s" % (
                "untimed cache reset + prefill" if hbm else "cache reset + prefill", w.n_steps,
                ", each followed by the frozen-eviction backward" if backward else ""),
        },
        "tflops": round(tflops, 3),
        "tokens_per_s": round(tokens_per_s, 1),
        "roofline": roof,
        # the whole step against the same peak (roofline.frac covers the attention kernel only)
        "step_roofline_frac": round(value / (PEAK_HBM_GBS if hbm else roof["peak"]), 4),
        **({"step_with_state": with_state} if hbm else {}),
        **({"backward_executed": {
            "kernels": "bwd_dq + bwd_dkdv + chunk reduce" + (" + undo + route" if rec else ""),
            "ms_per_step": round(step_ms["backward"], 3),
            "tflops": round(sum(1.4 * f for kind, f in fl if kind == "backward") / (step_ms["backward"] * 1e-3) / 1e12, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s (14 d flops executed per visible pair and query head)"}}
           if backward else {}),
        "breakdown_pass": {
            "source": "one extra pass after the timed region with every kernel bracketed by library "
                      "events (their records add ~1-3 us per launch); not the timed passes",
            "kernel_ms_per_step": {k: round(v, 4) for k, v in step_ms.items()}},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
