"""GPU parity of short-chunk H2O steps, whose attention and column masses run
in one kernel (at most 512 query rows G*S per KV group, in up to 16 parts of
32 rows; at most 72 blocks of 32 keys per head: the cache's, then the
chunk's), against the fp64 oracle: every step, every head.

Shapes cover 1, 2, 7, 9 and 16 row parts of a group, d = 64 and 128, filled
lengths that are not multiples of 32 (partial key blocks) through the fill
phase into eviction, both workgroup-to-head mappings (head counts that are and
are not multiples of 8), the largest cache the kernel takes and one slot more
(which runs the attention and score kernels instead), and an adopted state with
free slots inside the scanned range.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from kv_cache_eviction_amd import workloads as wl
from tests.parity_helpers import (assert_cuts_checked, assert_within, cfg_of, h2o_mod, merge_errors,
                                  run_and_check_step)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


SHAPES = {
    # two halves (64 rows), 4 heads (plain mapping), fill phase then eviction
    "g4_s16_d128_fill": dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, prefill=100, chunk=16,
                             total_len=100 + 16 * 12, cache_slots=200, recent_window=24, qk_std=1.0),
    # two halves, 8 heads (the two halves of a head 8 workgroups apart), d = 64
    "g8_s8_d64_h8": dict(batch=1, n_q_heads=64, n_kv_heads=8, head_dim=64, prefill=300, chunk=8,
                         total_len=300 + 8 * 8, cache_slots=330, recent_window=16, qk_std=1.0),
    # one half with rows past the end (6 rows), S = 3
    "g2_s3_d128": dict(batch=3, n_q_heads=4, n_kv_heads=2, head_dim=128, prefill=45, chunk=3,
                       total_len=45 + 3 * 12, cache_slots=60, recent_window=5, qk_std=1.0),
    # single-token steps, G = 1
    "g1_s1_d64": dict(batch=2, n_q_heads=2, n_kv_heads=2, head_dim=64, prefill=33, chunk=1,
                      total_len=33 + 1 * 16, cache_slots=40, recent_window=4, qk_std=1.0),
    # 16 row parts (128-token chunks, G = 4), 8 heads: each head's parts on one XCD
    "g4_s128_d128_h8": dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, prefill=256, chunk=128,
                            total_len=256 + 128 * 5, cache_slots=512, recent_window=64, qk_std=1.0),
    # 7 row parts, the last partial (200 rows)
    "g2_s100_d64": dict(batch=2, n_q_heads=4, n_kv_heads=2, head_dim=64, prefill=150, chunk=100,
                        total_len=150 + 100 * 4, cache_slots=300, recent_window=30, qk_std=1.0),
    # 9 row parts (264 rows): the select sums 9 splits
    "g8_s33_d128": dict(batch=1, n_q_heads=16, n_kv_heads=2, head_dim=128, prefill=100, chunk=33,
                        total_len=100 + 33 * 5, cache_slots=180, recent_window=20, qk_std=1.0),
    # the largest cache the fused kernel takes: 71 cache blocks of 32 slots and
    # the chunk's block, 72 = 8 waves x 9 blocks
    "g4_s16_m2272_d64": dict(batch=1, n_q_heads=4, n_kv_heads=1, head_dim=64, prefill=2272, chunk=16,
                             total_len=2272 + 16 * 4, cache_slots=2272, recent_window=32, qk_std=1.0),
    # one slot more: attention and score kernels
    "g4_s16_m2273_d64": dict(batch=1, n_q_heads=4, n_kv_heads=1, head_dim=64, prefill=2273, chunk=16,
                             total_len=2273 + 16 * 3, cache_slots=2273, recent_window=32, qk_std=1.0),
}


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_short_chunk_steps_every_step(name):
    h2o = h2o_mod()
    w = wl.workload("llama8b_64k", **SHAPES[name])
    cfg = cfg_of(w)
    cache = h2o.H2OCache(cfg)
    hh = wl.heavy_hitters(w, 5)
    heads = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    worst = {}
    for c in range(w.n_chunks):
        q, k, v = wl.chunk_inputs(w, 5, c, hh=hh)
        _say(f"[{name}] chunk {c}")
        errs = run_and_check_step(cache, cfg, q, k, v, heads, w.recent_window, prefill=(c == 0))
        assert_within(errs, f"{name} chunk {c}")
        merge_errors(worst, errs)
    torch.cuda.synchronize()
    assert h2o.h2o_device_status(cache.handle) == 0
    assert worst["evicting"] > 0
    assert_cuts_checked(worst, name)
    _say(f"[{name}] worst {worst}")


def test_adopted_state_with_free_slots():
    """Free slots (position -1) scattered through the scanned range: they are
    masked out of the attention and the masses, and filled first."""
    h2o = h2o_mod()
    w = wl.workload("llama8b_64k", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, prefill=16, chunk=16,
                    total_len=16 * 8, cache_slots=150, recent_window=20, qk_std=1.0)
    B, Hkv, M, d = w.batch, w.n_kv_heads, w.cache_slots, w.head_dim
    cfg = cfg_of(w)
    rng = np.random.default_rng(11)
    T = 1000
    pos = np.full((B, Hkv, M), -1, dtype=np.int32)
    scores = np.zeros((B, Hkv, M), dtype=np.float32)
    for b in range(B):
        for h in range(Hkv):
            filled = rng.choice(M, size=118, replace=False)
            pos[b, h, filled] = rng.choice(T, size=118, replace=False)
            scores[b, h, filled] = rng.uniform(0.1, 5.0, size=118).astype(np.float32)
    kv = rng.standard_normal((2, B, Hkv, M, d)).astype(np.float32)
    state = (torch.from_numpy(wl.to_bf16_bits(kv[0]).view(np.int16)).cuda().view(torch.bfloat16),
             torch.from_numpy(wl.to_bf16_bits(kv[1]).view(np.int16)).cuda().view(torch.bfloat16),
             torch.from_numpy(scores).cuda(), torch.from_numpy(pos).cuda())
    cache = h2o.H2OCache(cfg, adopt_state=state, tokens_seen=T)
    heads = [(b, h) for b in range(B) for h in range(Hkv)]
    worst = {}
    for c in range(1, w.n_chunks):
        q, k, v = wl.chunk_inputs(w, 9, c)
        _say(f"[free slots] chunk {c}")
        errs = run_and_check_step(cache, cfg, q, k, v, heads, w.recent_window)
        assert_within(errs, f"free slots chunk {c}")
        merge_errors(worst, errs)
    torch.cuda.synchronize()
    assert h2o.h2o_device_status(cache.handle) == 0
    # 32 free slots per head take the first two steps' tokens, then the cache evicts
    assert worst["evicting"] > 0
    _say(f"[free slots] worst {worst}")
