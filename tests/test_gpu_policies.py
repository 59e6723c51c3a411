"""GPU parity of the position eviction policies (recent, sink_recent: the
pages' lr and slr rows) against the fp64 oracle run free with the same
policy.  Positions are unique, so the decisions cannot tie: written slots and
the position array must match bit-exactly at every step; outputs use the
forward's bounds (max |dO| <= 2e-2, rel-RMS <= 5e-3) and lse max abs 1e-3.
No score is kept: the scores stay 0.  The S < 32 short-chunk path and
d = 64 are covered as well as a chunk longer than 1024 (the select kernel's
tail loop), and the fp32 path."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from kv_cache_eviction_amd import workloads as wl
from oracle import h2o_oracle as orc
from tests.parity_helpers import cfg_of, h2o_mod, to_device

pytestmark = pytest.mark.gpu

CASES = {
    "recent_g4_d128": ("recent", 0, dict(batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128, prefill=200,
                                         chunk=100, total_len=200 + 100 * 6, cache_slots=320,
                                         recent_window=40, qk_std=1.0)),
    "sink_recent_g2_d64_b2": ("sink_recent", 4, dict(batch=2, n_q_heads=4, n_kv_heads=2, head_dim=64,
                                                     prefill=96, chunk=64, total_len=96 + 64 * 6,
                                                     cache_slots=200, recent_window=16, qk_std=1.0)),
    "sink_recent_short_s12": ("sink_recent", 8, dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128,
                                                     prefill=64, chunk=12, total_len=64 + 12 * 8,
                                                     cache_slots=96, recent_window=8, qk_std=1.0)),
    "sink_recent_fp32_d64": ("sink_recent", 2, dict(batch=1, n_q_heads=4, n_kv_heads=2, head_dim=64,
                                                    dtype="fp32", prefill=64, chunk=32, total_len=64 + 32 * 6,
                                                    cache_slots=96, recent_window=8, qk_std=1.0)),
    "recent_long_chunk_1100": ("recent", 0, dict(batch=1, n_q_heads=2, n_kv_heads=1, head_dim=128,
                                                 prefill=1200, chunk=1100, total_len=1200 + 1100 * 3,
                                                 cache_slots=2400, recent_window=100, qk_std=1.0)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_position_policy_matches_oracle(name):
    policy, n_sink, kw = CASES[name]
    h2o = h2o_mod()
    w = wl.workload("llama8b_64k", **kw)
    cfg = cfg_of(w, policy=policy, n_sink=n_sink)
    cache = h2o.H2OCache(cfg)
    seed = 3
    hh = wl.heavy_hitters(w, seed)
    chunks = [wl.chunk_inputs(w, seed, c, hh=hh) for c in range(w.n_chunks)]
    f64 = [tuple(wl.stored_to_f64(x) for x in ch) for ch in chunks]
    _, hist = orc.run_sequence(f64, w.cache_slots, w.recent_window, 1.0 / math.sqrt(w.head_dim),
                               keep_history=True, policy=policy, n_sink=n_sink)
    assert any(len(e) for h in hist for per_b in h["evicted"] for e in per_b if e is not None)
    B, Hq, Hkv = w.batch, w.n_q_heads, w.n_kv_heads
    for c, (q, k, v) in enumerate(chunks):
        qt, kt, vt = to_device(q), to_device(k), to_device(v)
        n = qt.shape[2]
        lse = torch.empty((B, Hq, n), dtype=torch.float32, device="cuda")
        if c == 0:
            out = cache.prefill(qt, kt, vt, lse=lse)
        else:
            slots = torch.empty((B, Hkv, n), dtype=torch.int32, device="cuda")
            out = cache.chunk_step(qt, kt, vt, lse=lse, slots_out=slots)
        torch.cuda.synchronize()
        ref = hist[c]
        got = out.double().cpu().numpy()
        err = np.abs(got - ref["out"]).max()
        rel = np.linalg.norm(got - ref["out"]) / np.linalg.norm(ref["out"])
        assert err <= 2e-2 and rel <= 5e-3, (name, c, err, rel)
        assert np.abs(lse.double().cpu().numpy() - ref["lse"]).max() <= 1e-3, (name, c)
        if c > 0:
            assert (slots.cpu().numpy() == ref["targets"]).all(), (name, c)
        assert (cache.positions.cpu().numpy() == ref["pos"]).all(), (name, c)
        assert (cache.scores.cpu().numpy() == 0).all(), (name, c)
    print(f"[policy {name}] {w.n_chunks} chunks ok", flush=True)


def test_position_policy_rejects_step_mass():
    h2o = h2o_mod()
    _, _, kw = CASES["recent_g4_d128"]
    w = wl.workload("llama8b_64k", **kw)
    cache = h2o.H2OCache(cfg_of(w, policy="recent"))
    q, k, v = (to_device(x) for x in wl.chunk_inputs(w, 1, 0))
    cache.prefill(q, k, v)
    q, k, v = (to_device(x) for x in wl.chunk_inputs(w, 1, 1))
    mass = torch.empty((w.batch, w.n_kv_heads, w.cache_slots + q.shape[2]), dtype=torch.float32, device="cuda")
    with pytest.raises(h2o.H2OError) as e:
        cache.chunk_step(q, k, v, step_mass=mass)
    assert e.value.status == h2o.H2O_ERR_UNSUPPORTED
    assert cache.tokens_seen == w.prefill
