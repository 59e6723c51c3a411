"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Every checked step is teacher-forced: the oracle starts from the GPU's own
state before the step (exact in float64), so one near-tie at an eviction cut
cannot fork the rest of the comparison.  Sizes span several tiles and ragged
tails; the named workloads run at full size with sampled steps and heads.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from kv_cache_eviction_amd import workloads as wl
from oracle import h2o_oracle as orc
from tests.parity_helpers import (assert_cuts_checked, assert_within, cfg_of, merge_errors,
                                  run_and_check_step, snapshot, to_device, to_f64, h2o_mod)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _run(w: wl.Workload, seed: int, check_steps, heads, cfg_kw=None, max_steps=None):
    """Runs workload `w` on the GPU; checks the listed chunk indices (0 = prefill)."""
    h2o = h2o_mod()
    cfg = cfg_of(w, **(cfg_kw or {}))
    cache = h2o.H2OCache(cfg)
    hh = wl.heavy_hitters(w, seed)
    n_chunks = w.n_chunks if max_steps is None else min(w.n_chunks, max_steps + 1)
    worst = {}
    for c in range(n_chunks):
        q, k, v = wl.chunk_inputs(w, seed, c, hh=hh)
        if c in check_steps:
            _say(f"[{w.name}] check chunk {c}")
            errs = run_and_check_step(cache, cfg, q, k, v, heads, w.recent_window, prefill=(c == 0))
            assert_within(errs, f"{w.name} chunk {c}")
            merge_errors(worst, errs)
        else:
            qt, kt, vt = to_device(q), to_device(k), to_device(v)
            if c == 0:
                cache.prefill(qt, kt, vt)
            else:
                cache.chunk_step(qt, kt, vt)
    torch.cuda.synchronize()
    assert h2o.h2o_device_status(cache.handle) == 0
    _say(f"[{w.name}] worst errors {worst}")
    assert_cuts_checked(worst, w.name)
    return cache, worst


def _all_heads(w):
    return [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]


def test_tiny_fp32_every_step():
    w = wl.workload("tiny")
    _run(w, 0, set(range(w.n_chunks)), _all_heads(w))


@pytest.mark.parametrize("seed", [1, 2])
def test_tiny_fp32_other_seeds(seed):
    w = wl.workload("tiny")
    _run(w, seed, set(range(w.n_chunks)), _all_heads(w))


SMALL_BF16 = {
    # several tiles and ragged tails: S, N_C, M not multiples of 32/64
    "g4_d128_ragged": dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, prefill=200, chunk=100,
                           total_len=200 + 100 * 5, cache_slots=320, recent_window=40, qk_std=1.0),
    "g1_d64": dict(batch=1, n_q_heads=3, n_kv_heads=3, head_dim=64, prefill=130, chunk=70,
                   total_len=130 + 70 * 5, cache_slots=260, recent_window=17, qk_std=1.0),
    "g8_d128_fill": dict(batch=1, n_q_heads=16, n_kv_heads=2, head_dim=128, prefill=64, chunk=96,
                         total_len=64 + 96 * 7, cache_slots=512, recent_window=64, qk_std=1.0),
    "g2_small_chunks": dict(batch=3, n_q_heads=4, n_kv_heads=2, head_dim=128, prefill=96, chunk=5,
                            total_len=96 + 5 * 12, cache_slots=100, recent_window=9, qk_std=1.0),
    # short chunks (S < 32): rows of several heads packed into one row block
    "g8_short16": dict(batch=2, n_q_heads=16, n_kv_heads=2, head_dim=128, prefill=64, chunk=16,
                       total_len=64 + 16 * 8, cache_slots=128, recent_window=16, qk_std=1.0),
    "g4_short31_d64": dict(batch=1, n_q_heads=8, n_kv_heads=2, head_dim=64, prefill=70, chunk=31,
                           total_len=70 + 31 * 6, cache_slots=150, recent_window=20, qk_std=1.0),
    "g3_decode1": dict(batch=2, n_q_heads=6, n_kv_heads=2, head_dim=128, prefill=50, chunk=1,
                       total_len=50 + 1 * 20, cache_slots=60, recent_window=8, qk_std=1.0),
    "g1_short20": dict(batch=1, n_q_heads=2, n_kv_heads=2, head_dim=128, prefill=40, chunk=20,
                       total_len=40 + 20 * 5, cache_slots=80, recent_window=10, qk_std=1.0),
    # cache sizes that give the select pass 2 and 32 slots per thread
    "g2_m700_d64": dict(batch=1, n_q_heads=4, n_kv_heads=2, head_dim=64, prefill=600, chunk=64,
                        total_len=600 + 64 * 4, cache_slots=700, recent_window=50, qk_std=1.0),
    "g1_m8200_d64": dict(batch=1, n_q_heads=1, n_kv_heads=1, head_dim=64, prefill=8192, chunk=40,
                         total_len=8192 + 40 * 3, cache_slots=8200, recent_window=64, qk_std=1.0),
    # chunks of 257..4096 tokens: several select workgroups per head, each
    # copying a share of the rows (M and S multiples of 4) ...
    "g4_s300_parts": dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=64, prefill=320, chunk=300,
                          total_len=320 + 300 * 4, cache_slots=704, recent_window=40, qk_std=1.0),
    # ... or one select workgroup and the scatter kernel (S not a multiple of 4)
    "g2_s301_scatter": dict(batch=1, n_q_heads=4, n_kv_heads=2, head_dim=128, prefill=258, chunk=301,
                            total_len=258 + 301 * 4, cache_slots=700, recent_window=30, qk_std=1.0),
}


@pytest.mark.parametrize("name", sorted(SMALL_BF16))
def test_small_bf16_every_step(name):
    w = wl.workload("llama8b_64k", **SMALL_BF16[name])
    _run(w, 3, set(range(w.n_chunks)), _all_heads(w))


def test_cache_holding_everything_is_exact_causal_attention():
    """M >= L: no eviction ever, the output is causal attention over the sequence."""
    h2o = h2o_mod()
    w = wl.workload("llama8b_64k", batch=1, n_q_heads=8, n_kv_heads=2, prefill=160, chunk=96,
                    total_len=160 + 96 * 4, cache_slots=640, recent_window=32, qk_std=1.0)
    cfg = cfg_of(w)
    cache = h2o.H2OCache(cfg)
    outs, qs, ks, vs = [], [], [], []
    for c in range(w.n_chunks):
        q, k, v = wl.chunk_inputs(w, 5, c)
        qt, kt, vt = to_device(q), to_device(k), to_device(v)
        outs.append(cache.prefill(qt, kt, vt) if c == 0 else cache.chunk_step(qt, kt, vt))
        qs.append(qt.float().cpu()); ks.append(kt.float().cpu()); vs.append(vt.float().cpu())
    out = torch.cat([o.float().cpu() for o in outs], dim=2).double()
    q = torch.cat(qs, 2).double()
    G = w.group
    k = torch.cat(ks, 2).double().repeat_interleave(G, dim=1)
    v = torch.cat(vs, 2).double().repeat_interleave(G, dim=1)
    ref = F.scaled_dot_product_attention(q, k, v, is_causal=True)
    err = (out - ref).abs().max().item()
    rel = ((out - ref).norm() / ref.norm()).item()
    _say(f"exact-attention max abs {err:.3e} rel rms {rel:.3e}")
    assert err <= 2e-2 and rel <= 5e-3
    # every key's score is its full causal column mass
    L = q.shape[2]
    z = (q @ k.transpose(-1, -2)) / math.sqrt(w.head_dim)
    z = z.masked_fill(~torch.ones(L, L, dtype=torch.bool).tril(), float("-inf"))
    colmass = torch.softmax(z, -1).sum(2).reshape(1, w.n_kv_heads, G, L).sum(2)
    torch.cuda.synchronize()
    sig = cache.scores.double().cpu()[:, :, :L]
    assert (cache.positions.cpu()[:, :, :L] == torch.arange(L, dtype=torch.int32)).all()
    assert ((sig - colmass).abs() / colmass).max().item() <= 1e-3


def test_llama8b_64k_sampled_steps():
    w = wl.workload("llama8b_64k")
    _run(w, 0, {0, 1, 31, 62}, [(0, 0), (0, 5)])


def test_llama8b_64k_s128_sampled_steps():
    """128-token chunks: the attention splits each row group's keys over 4
    workgroups and merges them."""
    w = wl.workload("llama8b_64k_s128")
    _run(w, 0, {1, 2, 17, 250, 496}, [(0, 0), (0, 6)])


def test_llama8b_128k_sampled_steps():
    w = wl.workload("llama8b_128k")
    _run(w, 0, {1, 2, 3, 64, 126}, [(0, 3)])


def test_decode_b32_sampled_steps():
    w = wl.workload("decode_b32")
    _run(w, 0, {1, 128, 256}, [(0, 0), (17, 5), (31, 7)])


def test_widegqa_forward_sampled_steps():
    w = wl.workload("widegqa_128k")
    _run(w, 0, {1, 2, 3, 62}, [(0, 2)])


def _small_run(seed=7, steps=6):
    h2o = h2o_mod()
    w = wl.workload("llama8b_64k", **SMALL_BF16["g4_d128_ragged"])
    cfg = cfg_of(w)
    cache = h2o.H2OCache(cfg)
    outs = []
    for c in range(min(w.n_chunks, steps)):
        q, k, v = (to_device(x) for x in wl.chunk_inputs(w, seed, c))
        outs.append((cache.prefill(q, k, v) if c == 0 else cache.chunk_step(q, k, v)).cpu())
    torch.cuda.synchronize()
    return w, cfg, cache, outs


def test_bitwise_deterministic():
    _, _, a, oa = _small_run()
    _, _, b, ob = _small_run()
    for x, y in zip(oa, ob):
        assert torch.equal(x, y)
    for t in ("k_cache", "v_cache", "scores", "positions"):
        assert torch.equal(getattr(a, t).cpu(), getattr(b, t).cpu()), t


def test_resume_from_snapshot_equals_uninterrupted():
    h2o = h2o_mod()
    w, cfg, ref, ref_outs = _small_run(steps=6)
    # run 3 chunks, snapshot, destroy, adopt into fresh buffers, continue
    cache = h2o.H2OCache(cfg)
    outs = []
    for c in range(3):
        q, k, v = (to_device(x) for x in wl.chunk_inputs(w, 7, c))
        outs.append((cache.prefill(q, k, v) if c == 0 else cache.chunk_step(q, k, v)).cpu())
    torch.cuda.synchronize()
    state = tuple(t.clone() for t in (cache.k_cache, cache.v_cache, cache.scores, cache.positions))
    T = cache.tokens_seen
    cache.close()
    resumed = h2o.H2OCache(cfg, adopt_state=state, tokens_seen=T)
    for c in range(3, 6):
        q, k, v = (to_device(x) for x in wl.chunk_inputs(w, 7, c))
        outs.append(resumed.chunk_step(q, k, v).cpu())
    torch.cuda.synchronize()
    for x, y in zip(outs, ref_outs):
        assert torch.equal(x, y)
    for t in ("k_cache", "v_cache", "scores", "positions"):
        assert torch.equal(getattr(resumed, t).cpu(), getattr(ref, t).cpu()), t


def test_planted_exact_ties_evict_lowest_slots():
    """All candidates tie exactly: with Q = 0 every key gets the same mass, so
    the victims must be the lowest-index candidates, bit-exact."""
    h2o = h2o_mod()
    B, Hq, Hkv, d, M, S, W = 1, 4, 2, 128, 256, 32, 64
    cfg = h2o.H2OConfig(B, Hq, Hkv, d, M, W, S, M, "bf16")
    T = 1000
    pos = torch.empty((B, Hkv, M), dtype=torch.int32)
    for h in range(Hkv):
        pos[0, h] = torch.randperm(M, generator=torch.Generator().manual_seed(h)).to(torch.int32) + (T - M)
    k_cache = torch.randn((B, Hkv, M, d), generator=torch.Generator().manual_seed(9)).to(torch.bfloat16)
    state = (k_cache.cuda(), torch.randn_like(k_cache.float()).to(torch.bfloat16).cuda(),
             torch.full((B, Hkv, M), 2.5, dtype=torch.float32).cuda(), pos.cuda())
    cache = h2o.H2OCache(cfg, adopt_state=state, tokens_seen=T)
    q = torch.zeros((B, Hq, S, d), dtype=torch.bfloat16, device="cuda")
    k = torch.randn((B, Hkv, S, d), device="cuda").to(torch.bfloat16)
    v = torch.randn((B, Hkv, S, d), device="cuda").to(torch.bfloat16)
    slots = torch.empty((B, Hkv, S), dtype=torch.int32, device="cuda")
    cache.chunk_step(q, k, v, slots_out=slots)
    torch.cuda.synchronize()
    for h in range(Hkv):
        cand = np.flatnonzero(pos[0, h].numpy() < T - W)
        assert slots[0, h].cpu().numpy().tolist() == sorted(cand[:S].tolist())


def test_mass_per_step_is_chunk_times_group():
    h2o = h2o_mod()
    w = wl.workload("llama8b_64k", **SMALL_BF16["g8_d128_fill"])
    cfg = cfg_of(w)
    cache = h2o.H2OCache(cfg)
    for c in range(w.n_chunks):
        q, k, v = (to_device(x) for x in wl.chunk_inputs(w, 11, c))
        if c == 0:
            cache.prefill(q, k, v)
            continue
        mass = torch.empty((1, w.n_kv_heads, w.cache_slots + w.chunk), device="cuda")
        cache.chunk_step(q, k, v, step_mass=mass)
        tot = mass.double().sum(-1).cpu()
        assert torch.allclose(tot, torch.full_like(tot, w.chunk * w.group), rtol=1e-5), tot


def test_error_paths_leave_state_unchanged():
    h2o = h2o_mod()
    w = wl.workload("llama8b_64k", **SMALL_BF16["g2_small_chunks"])
    cfg = cfg_of(w)
    cache = h2o.H2OCache(cfg)
    q, k, v = (to_device(x) for x in wl.chunk_inputs(w, 1, 0))
    cache.prefill(q, k, v)
    with pytest.raises(h2o.H2OError) as e:
        cache.prefill(q, k, v)                   # second prefill
    assert e.value.status == h2o.H2O_ERR_STATE
    q1, k1, v1 = (to_device(x) for x in wl.chunk_inputs(w, 1, 1))
    big = torch.zeros((w.batch, w.n_q_heads, w.chunk + 1, w.head_dim), dtype=torch.bfloat16, device="cuda")
    bigkv = torch.zeros((w.batch, w.n_kv_heads, w.chunk + 1, w.head_dim), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(h2o.H2OError) as e:
        cache.chunk_step(big, bigkv, bigkv)      # s > max_chunk
    assert e.value.status == h2o.H2O_ERR_SHAPE
    rc = h2o._lib.h2o_chunk_step(cache.handle, None, None, None, 4, None, None, None, None, None, None, None,
                                 None)
    assert rc == h2o.H2O_ERR_NULL
    # a query buffer 8 bytes off a 16-byte boundary: refused before any launch
    flat = torch.empty(q1.numel() + 8, dtype=torch.bfloat16, device="cuda")
    q_off = flat[4:4 + q1.numel()].view(q1.shape)
    q_off.copy_(q1)
    with pytest.raises(ValueError):
        cache.chunk_step(q_off, k1, v1)
    out = torch.empty_like(q1)
    rc = h2o._lib.h2o_chunk_step(cache.handle, q_off.data_ptr(), k1.data_ptr(), v1.data_ptr(), w.chunk,
                                 out.data_ptr(), None, None, None, None, None, None, None)
    assert rc == h2o.H2O_ERR_ALIGN
    assert cache.tokens_seen == w.prefill
    cache.chunk_step(q1, k1, v1)
    assert cache.tokens_seen == w.prefill + w.chunk


def test_scores_snapshot_and_timing_counters():
    """h2o_get_scores copies the live scores and positions; the event timing
    counts exactly the launches of the selected kernels."""
    h2o = h2o_mod()
    w = wl.workload("llama8b_64k", **SMALL_BF16["g4_d128_ragged"])
    cache = h2o.H2OCache(cfg_of(w))
    h2o.h2o_set_timing(cache.handle, ["attn_fwd", "select"])
    steps = 4
    for c in range(steps):
        q, k, v = (to_device(x) for x in wl.chunk_inputs(w, 2, c))
        if c == 0:
            cache.prefill(q, k, v)
        else:
            cache.chunk_step(q, k, v)
    sc, ps = cache.get_scores()
    torch.cuda.synchronize()
    assert torch.equal(sc, cache.scores) and torch.equal(ps, cache.positions)
    for name in ("attn_fwd", "select"):
        ms, n = h2o.h2o_get_timing(cache.handle, name)
        assert n == steps and ms > 0, (name, ms, n)
    assert h2o.h2o_get_timing(cache.handle, "score") == (0.0, 0)
    with pytest.raises(h2o.H2OError) as e:
        h2o.h2o_get_timing(cache.handle, 7)
    assert e.value.status == h2o.H2O_ERR_SHAPE


@pytest.mark.parametrize("S,M", [(16, 64), (300, 640), (4160, 4352)])
def test_infeasible_adopted_state_sets_device_status(S, M):
    """An adopted state with nothing evictable: no slot is written, the status
    bit is set, and every optional output is still defined (S = 16: one
    select workgroup per head handles the rows; S = 300: several select
    parts per head; S = 4160: the scatter kernel)."""
    h2o = h2o_mod()
    B, Hq, Hkv, d, W = 1, 2, 1, 64, 8
    cfg = h2o.H2OConfig(B, Hq, Hkv, d, M, W, S, M, "bf16")
    T = 1000
    # every slot inside the recent window: nothing is evictable
    pos = torch.full((B, Hkv, M), T - 1, dtype=torch.int32)
    state = (torch.zeros((B, Hkv, M, d), dtype=torch.bfloat16).cuda(),
             torch.zeros((B, Hkv, M, d), dtype=torch.bfloat16).cuda(),
             torch.ones((B, Hkv, M), dtype=torch.float32).cuda(), pos.cuda())
    before = tuple(t.clone() for t in state)
    cache = h2o.H2OCache(cfg, adopt_state=state, tokens_seen=T)
    q = torch.randn((B, Hq, S, d), device="cuda").to(torch.bfloat16)
    k = torch.randn((B, Hkv, S, d), device="cuda").to(torch.bfloat16)
    # optional outputs pre-filled with garbage: all must be overwritten
    slots = torch.full((B, Hkv, S), 7, dtype=torch.int32, device="cuda")
    pos_old = torch.full((B, Hkv, S), 7, dtype=torch.int32, device="cuda")
    mass = torch.full((B, Hkv, M + S), -5.0, dtype=torch.float32, device="cuda")
    k_old = torch.full((B, Hkv, S, d), 3.0, dtype=torch.bfloat16, device="cuda")
    v_old = torch.full_like(k_old, 3.0)
    cache.chunk_step(q, k, k.clone(), slots_out=slots, step_mass=mass, k_old=k_old, v_old=v_old,
                     pos_old=pos_old)
    assert h2o.h2o_device_status(cache.handle) == 1
    assert h2o.h2o_device_status(cache.handle) == 0         # cleared by the read
    # no slot written; the scores received the step's (positive) mass
    for i in (0, 1, 3):
        assert torch.equal(before[i], state[i])
    assert (state[2] > before[2]).all()
    assert (slots == -1).all() and (pos_old == -1).all()
    assert (k_old.float() == 0).all() and (v_old.float() == 0).all()
    m = mass.double().cpu()
    assert (m > 0).all()
    assert torch.allclose(m.sum(-1), torch.full((B, Hkv), float(S * Hq // Hkv), dtype=torch.float64), rtol=1e-5)
    assert torch.allclose(m[..., :M], (state[2] - before[2]).double().cpu(), rtol=1e-6, atol=0)


@pytest.mark.parametrize("name,overrides", [
    ("llama8b_64k", dict(total_len=2048 + 1024 * 3)),            # long-chunk forward
    ("decode_b32", dict(batch=4, total_len=2048 + 16 * 6)),        # fused short-chunk kernel
    ("llama8b_64k_s128", dict(total_len=2048 + 128 * 4)),          # fused kernel, 16 row parts
])
def test_filled_cache_attention_equals_the_general_one(name, overrides):
    """Once the cache has filled, the forward (and the fused short-chunk
    kernel) skips the per-tile position copies; an adopted copy of the same
    state (whose fill the library cannot know) takes the general kernels.
    The two must agree bit for bit: every output, logsumexp and the final
    state."""
    h2o = h2o_mod()
    w = wl.workload(name, **overrides)
    cfg = cfg_of(w)
    hh = wl.heavy_hitters(w, 0)
    chunks = [tuple(to_device(x) for x in wl.chunk_inputs(w, 0, c, hh=hh)) for c in range(w.n_chunks)]

    def steps(cache):
        res = []
        for q, k, v in chunks[1:]:
            lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
            out = cache.chunk_step(q, k, v, lse=lse)
            res.append((out, lse))
        torch.cuda.synchronize()
        return res

    filled = h2o.H2OCache(cfg)
    filled.prefill(*chunks[0])
    torch.cuda.synchronize()
    state = tuple(t.clone() for t in (filled.k_cache, filled.v_cache, filled.scores, filled.positions))
    assert int(state[3].min()) >= 0                   # the prefill filled every slot
    adopted = h2o.H2OCache(cfg, adopt_state=state, tokens_seen=filled.tokens_seen)
    a, b = steps(filled), steps(adopted)
    for c, ((o1, l1), (o2, l2)) in enumerate(zip(a, b)):
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), ("out", c)
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), ("lse", c)
    for t in ("k_cache", "v_cache", "scores", "positions"):
        x, y = getattr(filled, t), getattr(adopted, t)
        bits = torch.int16 if x.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(x.view(bits), y.view(bits)), t
