"""h2o_chunk_backward_static (no workspace, no allocation) against
h2o_chunk_backward on the same pre-step states: two calls in a row, the
second with a smaller chunk, must give bit-identical gradients (the same
deterministic kernels; the second call finds the first one's data in the
shared static scratch).  A request larger than the static scratch is refused
before anything is enqueued."""
from __future__ import annotations

import sys

import pytest
import torch

from kv_cache_eviction_amd import workloads as wl
from tests.parity_helpers import cfg_of, h2o_mod, to_device

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _backward_both(h2o, cfg, state, q, k, v, out, lse, dO):
    Kc, Vc, pos = state
    res = []
    for static in (False, True):
        g = [torch.full_like(q, 5.0), torch.full_like(Kc, 5.0), torch.full_like(Vc, 5.0),
             torch.full_like(k, 5.0), torch.full_like(v, 5.0)]
        if static:
            h2o.h2o_chunk_backward_static(cfg, q, Kc, Vc, pos, k, v, out, lse, dO, *g)
        else:
            ws = torch.empty(h2o.h2o_backward_workspace_bytes(cfg, q.shape[2]), dtype=torch.uint8,
                             device="cuda")
            h2o.h2o_chunk_backward(cfg, q, Kc, Vc, pos, k, v, out, lse, dO, *g, ws)
        torch.cuda.synchronize()
        res.append([t.cpu() for t in g])
    return res


def test_static_scratch_backward_equals_workspace_backward():
    h2o = h2o_mod()
    w = wl.workload("widegqa_128k", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, prefill=200,
                    chunk=200, total_len=200 + 200 * 4, cache_slots=480, recent_window=40, qk_std=1.0)
    cfg = cfg_of(w)
    cache = h2o.H2OCache(cfg)
    hh = wl.heavy_hitters(w, 3)
    B, Hq, Hkv = w.batch, w.n_q_heads, w.n_kv_heads
    calls = 0
    for c in range(w.n_chunks):
        q, k, v = (to_device(x) for x in wl.chunk_inputs(w, 3, c, hh=hh))
        if c == 0:
            cache.prefill(q, k, v)
            continue
        # steps 3 (200 tokens, cache full: evicting) and 4 (cut to 70 tokens) are checked
        if c == 4:
            q, k, v = (t[:, :, :70].contiguous() for t in (q, k, v))
        if c < 3:
            cache.chunk_step(q, k, v)
            continue
        torch.cuda.synchronize()
        state = (cache.k_cache.clone(), cache.v_cache.clone(), cache.positions.clone())
        n = q.shape[2]
        lse = torch.empty((B, Hq, n), dtype=torch.float32, device="cuda")
        out = cache.chunk_step(q, k, v, lse=lse)
        dO = to_device(wl.chunk_grad_out(w, 3, c))[:, :, :n].contiguous()
        _say(f"[no-alloc backward] chunk {c}, s = {n}")
        ref, got = _backward_both(h2o, cfg, state, q, k, v, out, lse, dO)
        for name, a, b in zip(("dq", "dk_cache", "dv_cache", "dk_new", "dv_new"), ref, got):
            assert torch.equal(a, b), (c, name)
            assert torch.isfinite(a.float()).all(), (c, name)
        assert not torch.equal(ref[1], torch.full_like(ref[1], 5.0))
        calls += 1
    assert calls == 2


def test_static_scratch_refuses_requests_above_its_size():
    h2o = h2o_mod()
    B, Hq, Hkv, d, M, s = 1, 64, 8, 128, 4096, 4096      # needs 128.5 MiB of scratch
    cfg = h2o.H2OConfig(B, Hq, Hkv, d, M, 0, s, M, "bf16")
    assert h2o.h2o_backward_workspace_bytes(cfg, s) > 72 << 20
    z = lambda *shape: torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    q, out, dO, dq = (z(B, Hq, s, d) for _ in range(4))
    Kc, Vc, dKc, dVc = (z(B, Hkv, M, d) for _ in range(4))
    k, v, dk, dv = (z(B, Hkv, s, d) for _ in range(4))
    pos = torch.zeros((B, Hkv, M), dtype=torch.int32, device="cuda")
    lse = torch.zeros((B, Hq, s), dtype=torch.float32, device="cuda")
    with pytest.raises(h2o.H2OError) as e:
        h2o.h2o_chunk_backward_static(cfg, q, Kc, Vc, pos, k, v, out, lse, dO, dq, dKc, dVc, dk, dv)
    assert e.value.status == h2o.H2O_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert (dq == 0).all() and (dKc == 0).all()       # nothing was enqueued
