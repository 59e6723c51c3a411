"""GPU parity of the backward walk through the KV buffer over a row of chunks
(h2o_chunk_step's delta outputs + h2o_recurrence_backward_step) against the
fp64 oracle oracle/recurrence_grad.py (torch autograd through the unrolled
row with the eviction decisions held fixed).

The GPU run's eviction decisions must equal the oracle's own (bit-exact slot
ids; the seeds below have no near-tie at any cut).  Per chunk, the query
gradient and the total key/value gradients (own step plus every later step
that read the token's slot) are compared with rel-RMS <= 5e-3 and
max |err| <= 2e-2 * max |ref|, the bounds of the single-step backward.
Undoing every step, the prefill last, must give back the empty cache
exactly.  The walk carries every gradient in fp32 (no per-step rounding), so
the bound holds on rows of 20 and 30 steps as on short ones."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from kv_cache_eviction_amd import workloads as wl
from oracle import h2o_oracle as orc
from oracle import recurrence_grad as rg
from tests.parity_helpers import cfg_of, h2o_mod, to_device

pytestmark = pytest.mark.gpu

REL_RMS = 5e-3
MAX_REL = 2e-2

CASES = {
    "g2_d128": dict(batch=1, n_q_heads=4, n_kv_heads=2, head_dim=128, prefill=96, chunk=48,
                    total_len=96 + 48 * 5, cache_slots=160, recent_window=16, qk_std=1.0),
    "g4_d64_b2": dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=64, prefill=64, chunk=40,
                      total_len=64 + 40 * 5, cache_slots=128, recent_window=8, qk_std=1.0),
    # a long row: 20 chunk steps (4 fill steps, then 16 evicting), M = 1024
    "g4_d128_m1024_20steps": dict(batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128, prefill=512,
                                  chunk=128, total_len=512 + 128 * 20, cache_slots=1024,
                                  recent_window=128, qk_std=1.0),
    # 30 chunk steps at G = 8, d = 64, two sequences
    "g8_d64_b2_30steps": dict(batch=2, n_q_heads=16, n_kv_heads=2, head_dim=64, prefill=256, chunk=64,
                              total_len=256 + 64 * 30, cache_slots=512, recent_window=64, qk_std=1.0),
}


def _forward(w, seed):
    """GPU forward over the row with every step's delta recorded."""
    h2o = h2o_mod()
    cfg = cfg_of(w)
    cache = h2o.H2OCache(cfg)
    hh = wl.heavy_hitters(w, seed)
    B, Hq, Hkv, d = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    steps = []
    for c in range(w.n_chunks):
        q, k, v = (to_device(x) for x in wl.chunk_inputs(w, seed, c, hh=hh))
        n = q.shape[2]
        lse = torch.empty((B, Hq, n), dtype=torch.float32, device="cuda")
        if c == 0:
            out = cache.prefill(q, k, v, lse=lse)
            slots = torch.arange(n, dtype=torch.int32, device="cuda").expand(B, Hkv, n).contiguous()
            k_old = torch.zeros_like(k)
            v_old = torch.zeros_like(v)
            pos_old = torch.full((B, Hkv, n), -1, dtype=torch.int32, device="cuda")
        else:
            slots = torch.empty((B, Hkv, n), dtype=torch.int32, device="cuda")
            k_old, v_old = torch.empty_like(k), torch.empty_like(v)
            pos_old = torch.empty((B, Hkv, n), dtype=torch.int32, device="cuda")
            out = cache.chunk_step(q, k, v, lse=lse, slots_out=slots, k_old=k_old, v_old=v_old,
                                   pos_old=pos_old)
        dO = to_device(wl.chunk_grad_out(w, seed, c))
        steps.append(dict(q=q, k=k, v=v, out=out, lse=lse, dO=dO, slots=slots, k_old=k_old,
                          v_old=v_old, pos_old=pos_old))
    torch.cuda.synchronize()
    return cfg, cache, steps, hh


def _walk(cfg, cache, steps):
    """GPU backward walk, last step first; returns (dq, gk, gv) per chunk."""
    h2o = h2o_mod()
    B, Hkv, M, d = cfg.batch, cfg.n_kv_heads, cfg.cache_slots, cfg.head_dim
    kc, vc, pos = cache.k_cache.clone(), cache.v_cache.clone(), cache.positions.clone()
    acc_k = torch.zeros((B, Hkv, M, d), dtype=torch.float32, device="cuda")
    acc_v = torch.zeros_like(acc_k)
    s_max = max(st["q"].shape[2] for st in steps)
    ws = torch.empty(h2o.h2o_recurrence_workspace_bytes(cfg, s_max), dtype=torch.uint8, device="cuda")
    grads = [None] * len(steps)
    for c in reversed(range(len(steps))):
        st = steps[c]
        dq = torch.empty_like(st["q"])
        gk = torch.empty(st["k"].shape, dtype=torch.float32, device="cuda")
        gv = torch.empty_like(gk)
        h2o.h2o_recurrence_backward_step(cfg, kc, vc, pos, st["slots"], st["k_old"], st["v_old"],
                                         st["pos_old"], st["q"], st["k"], st["v"], st["out"], st["lse"],
                                         st["dO"], acc_k, acc_v, dq, gk, gv, ws)
        grads[c] = (dq, gk, gv)
    torch.cuda.synchronize()
    return kc, vc, pos, [tuple(t.double().cpu().numpy() for t in g) for g in grads]


@pytest.mark.parametrize("name", sorted(CASES))
def test_recurrence_gradients_match_oracle(name):
    w = wl.workload("widegqa_128k", **CASES[name])
    seed = 5
    cfg, cache, steps, hh = _forward(w, seed)
    # the oracle's own run: the same decisions, and its gradient through the row
    chunks = [tuple(wl.stored_to_f64(x) for x in wl.chunk_inputs(w, seed, c, hh=hh)) for c in range(w.n_chunks)]
    d_outs = [wl.stored_to_f64(wl.chunk_grad_out(w, seed, c)) for c in range(w.n_chunks)]
    scale = 1.0 / math.sqrt(w.head_dim)
    _, hist = orc.run_sequence(chunks, w.cache_slots, w.recent_window, scale, keep_history=True)
    targets = [h["targets"] for h in hist]
    for c in range(1, w.n_chunks):
        assert (steps[c]["slots"].cpu().numpy() == targets[c]).all(), f"chunk {c}: written slots differ"
    assert any(len(e) for h in hist for per_b in h["evicted"] for e in per_b if e is not None)
    ref = rg.row_grads(chunks, d_outs, targets, w.cache_slots, scale)

    kc, vc, pos, got = _walk(cfg, cache, steps)
    # every step undone: the empty cache the row started from
    assert (pos == -1).all()
    assert (kc.float() == 0).all() and (vc.float() == 0).all()
    worst = 0.0
    for c in range(w.n_chunks):
        for what, g, r in zip(("dq", "dk", "dv"), got[c], ref[c]):
            rel_rms = np.linalg.norm(g - r) / np.linalg.norm(r)
            max_rel = np.abs(g - r).max() / np.abs(r).max()
            worst = max(worst, rel_rms)
            assert rel_rms <= REL_RMS and max_rel <= MAX_REL, (name, c, what, rel_rms, max_rel)
    print(f"[recurrence {name}] {w.n_chunks} chunks, worst rel-rms {worst:.2e}", flush=True)


def test_recurrence_step_is_deterministic_and_validates():
    h2o = h2o_mod()
    w = wl.workload("widegqa_128k", **CASES["g2_d128"])
    cfg, cache, steps, _ = _forward(w, 6)
    runs = []
    for _ in range(2):
        _, _, _, g = _walk(cfg, cache, steps)
        runs.append(g)
    for a, b in zip(*runs):
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
    st = steps[-1]
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    acc = torch.zeros((w.batch, w.n_kv_heads, w.cache_slots, w.head_dim), dtype=torch.float32, device="cuda")
    gk = torch.empty(st["k"].shape, dtype=torch.float32, device="cuda")
    with pytest.raises(h2o.H2OError) as e:
        h2o.h2o_recurrence_backward_step(cfg, cache.k_cache, cache.v_cache, cache.positions, st["slots"],
                                         st["k_old"], st["v_old"], st["pos_old"], st["q"], st["k"], st["v"],
                                         st["out"], st["lse"], st["dO"], acc, acc.clone(),
                                         torch.empty_like(st["q"]), gk, gk.clone(), small)
    assert e.value.status == h2o.H2O_ERR_WORKSPACE
