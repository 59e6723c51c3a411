"""GPU parity of the frozen-eviction backward (h2o_chunk_backward) against the
fp64 oracle's textbook gradient, on the pre-step state of a real run.

Tolerances per gradient tensor: rel-RMS <= 5e-3 and max |err| <= 2e-2 *
max |ref| (the forward's output bounds applied relative to each tensor's
scale; gradients are written in bf16)."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from kv_cache_eviction_amd import workloads as wl
from oracle import h2o_oracle as orc
from tests.parity_helpers import cfg_of, h2o_mod, to_device

pytestmark = pytest.mark.gpu

REL_RMS = 5e-3
MAX_REL = 2e-2


def _grads_vs_oracle(w, cfg, state, q, k, v, out, lse, dO, heads):
    """Runs the backward on the GPU and compares the (b, kv head) pairs in `heads`."""
    h2o = h2o_mod()
    Kc, Vc, pos = state
    dq = torch.empty_like(q)
    dkc = torch.empty_like(Kc)
    dvc = torch.empty_like(Vc)
    dkn = torch.empty_like(k)
    dvn = torch.empty_like(v)
    ws = torch.empty(h2o.h2o_backward_workspace_bytes(cfg, q.shape[2]), dtype=torch.uint8, device="cuda")
    h2o.h2o_chunk_backward(cfg, q, Kc, Vc, pos, k, v, out, lse, dO, dq, dkc, dvc, dkn, dvn, ws)
    torch.cuda.synchronize()
    f = lambda t: t.double().cpu().numpy()
    Kn, Vn, Pn = f(Kc), f(Vc), pos.cpu().numpy().astype(np.int64)
    qn, kn, vn, gn = f(q), f(k), f(v), f(dO)
    gpu = [f(dq), f(dkc), f(dvc), f(dkn), f(dvn)]
    G = w.group
    worst = 0.0
    for b, h in heads:
        hs = slice(h * G, (h + 1) * G)
        hk = slice(h, h + 1)
        ref = orc.chunk_backward(Kn[b:b + 1, hk], Vn[b:b + 1, hk], Pn[b:b + 1, hk], qn[b:b + 1, hs],
                                 kn[b:b + 1, hk], vn[b:b + 1, hk], gn[b:b + 1, hs], 1.0 / math.sqrt(w.head_dim))
        got = [gpu[0][b:b + 1, hs]] + [t[b:b + 1, hk] for t in gpu[1:]]
        for name, g, r in zip(["dq", "dk_cache", "dv_cache", "dk_new", "dv_new"], got, ref):
            scale = np.abs(r).max()
            if scale == 0:
                assert np.abs(g).max() == 0, name
                continue
            rel_rms = np.linalg.norm(g - r) / np.linalg.norm(r)
            max_rel = np.abs(g - r).max() / scale
            worst = max(worst, rel_rms)
            assert rel_rms <= REL_RMS and max_rel <= MAX_REL, (name, b, h, rel_rms, max_rel)
        free = Pn[b, h] < 0
        assert (gpu[1][b, h][free] == 0).all() and (gpu[2][b, h][free] == 0).all()
    return worst


def _run_to(w, seed, step):
    """GPU run of workload `w` up to (excluding) chunk `step`; returns the cache."""
    h2o = h2o_mod()
    cfg = cfg_of(w)
    cache = h2o.H2OCache(cfg)
    hh = wl.heavy_hitters(w, seed)
    for c in range(step):
        q, k, v = (to_device(x) for x in wl.chunk_inputs(w, seed, c, hh=hh))
        if c == 0:
            cache.prefill(q, k, v)
        else:
            cache.chunk_step(q, k, v)
    return cfg, cache, hh


BWD_SMALL = {
    "g4_ragged_fill": dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, prefill=200, chunk=100,
                           total_len=200 + 100 * 5, cache_slots=320, recent_window=40, qk_std=1.0),
    "g8_d128": dict(batch=1, n_q_heads=16, n_kv_heads=2, head_dim=128, prefill=256, chunk=160,
                    total_len=256 + 160 * 4, cache_slots=384, recent_window=64, qk_std=1.0),
    "g1_d64": dict(batch=1, n_q_heads=3, n_kv_heads=3, head_dim=64, prefill=130, chunk=70,
                   total_len=130 + 70 * 5, cache_slots=260, recent_window=17, qk_std=1.0),
    # 6 needed rows per chunk tile: some of the 4 row pieces are empty
    "g2_tiny_chunk3": dict(batch=1, n_q_heads=4, n_kv_heads=2, head_dim=128, prefill=40, chunk=3,
                           total_len=40 + 3 * 5, cache_slots=48, recent_window=4, qk_std=1.0),
    # d = 64, three chunk tiles whose row pieces cross query-head boundaries
    "g4_d64_three_tiles": dict(batch=1, n_q_heads=8, n_kv_heads=2, head_dim=64, prefill=256, chunk=300,
                               total_len=256 + 300 * 4, cache_slots=640, recent_window=64, qk_std=1.0),
}


@pytest.mark.parametrize("name", sorted(BWD_SMALL))
@pytest.mark.parametrize("step", [1, 3])
def test_backward_small(name, step):
    w = wl.workload("widegqa_128k", **BWD_SMALL[name])
    cfg, cache, hh = _run_to(w, 4, step)
    torch.cuda.synchronize()
    state = (cache.k_cache.clone(), cache.v_cache.clone(), cache.positions.clone())
    q, k, v = (to_device(x) for x in wl.chunk_inputs(w, 4, step, hh=hh))
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    out = cache.chunk_step(q, k, v, lse=lse)
    dO = to_device(wl.chunk_grad_out(w, 4, step))
    worst = _grads_vs_oracle(w, cfg, state, q, k, v, out, lse, dO,
                             [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)])
    print(f"[bwd {name} step {step}] worst rel-rms {worst:.2e}", flush=True)


def test_backward_widegqa_sampled():
    w = wl.workload("widegqa_128k")
    step = 3                                   # the first step that evicts
    cfg, cache, hh = _run_to(w, 0, step)
    torch.cuda.synchronize()
    state = (cache.k_cache.clone(), cache.v_cache.clone(), cache.positions.clone())
    q, k, v = (to_device(x) for x in wl.chunk_inputs(w, 0, step, hh=hh))
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    out = cache.chunk_step(q, k, v, lse=lse)
    dO = to_device(wl.chunk_grad_out(w, 0, step))
    worst = _grads_vs_oracle(w, cfg, state, q, k, v, out, lse, dO, [(0, 5)])
    print(f"[bwd widegqa_128k step {step}] worst rel-rms {worst:.2e}", flush=True)


def test_backward_is_deterministic_and_validates():
    h2o = h2o_mod()
    w = wl.workload("widegqa_128k", **BWD_SMALL["g8_d128"])
    cfg, cache, hh = _run_to(w, 2, 2)
    torch.cuda.synchronize()
    Kc, Vc, pos = cache.k_cache.clone(), cache.v_cache.clone(), cache.positions.clone()
    q, k, v = (to_device(x) for x in wl.chunk_inputs(w, 2, 2, hh=hh))
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    out = cache.chunk_step(q, k, v, lse=lse)
    dO = to_device(wl.chunk_grad_out(w, 2, 2))
    ws = torch.empty(h2o.h2o_backward_workspace_bytes(cfg, q.shape[2]), dtype=torch.uint8, device="cuda")
    runs = []
    for _ in range(2):
        o = [torch.empty_like(t) for t in (q, Kc, Vc, k, v)]
        h2o.h2o_chunk_backward(cfg, q, Kc, Vc, pos, k, v, out, lse, dO, *o, ws)
        runs.append([t.cpu() for t in o])
    for a, b in zip(*runs):
        assert torch.equal(a, b)
    small_ws = ws[:16]
    with pytest.raises(h2o.H2OError) as e:
        h2o.h2o_chunk_backward(cfg, q, Kc, Vc, pos, k, v, out, lse, dO,
                               *[torch.empty_like(t) for t in (q, Kc, Vc, k, v)], small_ws)
    assert e.value.status == h2o.H2O_ERR_WORKSPACE
