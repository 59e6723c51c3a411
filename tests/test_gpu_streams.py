"""Independent caches on separate streams.

Every (sequence, KV head) pair of an H2O cache runs its own eviction, so a
batch can be served as several caches, each driven on its own HIP stream
with the library's calls interleaved on the host and the kernels of the
streams free to overlap on the GPU.  The library keeps no state outside its
handles, the caller's buffers and the workspace, so two such caches must
give, sequence for sequence and head for head, exactly what one cache over
the whole batch gives.  On the short-chunk path (attention and column
masses in one kernel, whose row parts depend only on G * S) the launch
shapes per head do not depend on the batch or the head count either, so the
comparison is bit for bit: every step's output and logsumexp, and the final
K/V cache, scores and positions.
"""
from __future__ import annotations

import pytest
import torch

from kv_cache_eviction_amd import workloads as wl
from tests.parity_helpers import cfg_of, h2o_mod, to_device

pytestmark = pytest.mark.gpu

CASES = {
    # decode-shaped: 16-token chunks, 4 sequences split 2 + 2 (the prefill's
    # G * N_C = 512 rows also take the short-chunk kernel)
    "decode_b4_batch_split": (dict(batch=4, n_q_heads=8, n_kv_heads=2, head_dim=128, prefill=128, chunk=16,
                                   total_len=128 + 16 * 16, cache_slots=256, recent_window=32), "batch"),
    # one sequence, its 4 KV heads split 2 + 2, 64-token chunks at d = 64
    "s64_b1_head_split": (dict(batch=1, n_q_heads=16, n_kv_heads=4, head_dim=64, prefill=128, chunk=64,
                               total_len=128 + 64 * 6, cache_slots=192, recent_window=16), "heads"),
}


def _views(t, g, n_groups, split):
    """Group g's part of a [B, H, ...] tensor: a contiguous slice of the
    batch, or (one sequence) of the heads."""
    if split == "batch":
        per = t.shape[0] // n_groups
        return t[g * per:(g + 1) * per]
    per = t.shape[1] // n_groups
    return t[:, g * per:(g + 1) * per]


def _run(w, seed, n_groups, split):
    h2o = h2o_mod()
    hh = wl.heavy_hitters(w, seed)
    chunks = [tuple(to_device(x) for x in wl.chunk_inputs(w, seed, c, hh=hh)) for c in range(w.n_chunks)]
    outs = [torch.full_like(q, float("nan")) for q, _, _ in chunks]
    lses = [torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda") for q, _, _ in chunks]
    if split == "batch":
        cfg = cfg_of(w, batch=w.batch // n_groups)
    else:
        cfg = cfg_of(w, n_q_heads=w.n_q_heads // n_groups, n_kv_heads=w.n_kv_heads // n_groups)
    caches = [h2o.H2OCache(cfg) for _ in range(n_groups)]
    streams = [torch.cuda.Stream() for _ in range(n_groups)] if n_groups > 1 else [torch.cuda.current_stream()]
    torch.cuda.synchronize()
    for c in range(w.n_chunks):
        q, k, v = chunks[c]
        for g in range(n_groups):
            gq, gk, gv = (_views(t, g, n_groups, split) for t in (q, k, v))
            go, gl = _views(outs[c], g, n_groups, split), _views(lses[c], g, n_groups, split)
            if c == 0:
                caches[g].prefill(gq, gk, gv, out=go, lse=gl, stream=streams[g])
            else:
                caches[g].chunk_step(gq, gk, gv, out=go, lse=gl, stream=streams[g])
    torch.cuda.synchronize()
    dim = 0 if split == "batch" else 1
    state = [torch.cat([getattr(cc, name) for cc in caches], dim=dim)
             for name in ("k_cache", "v_cache", "scores", "positions")]
    for cc in caches:
        assert h2o.h2o_device_status(cc.handle) == 0
        cc.close()
    return outs, lses, state


@pytest.mark.parametrize("name", sorted(CASES))
def test_two_caches_on_two_streams_equal_one_cache(name):
    shape, split = CASES[name]
    w = wl.workload("decode_b32", **shape)
    seed = 3
    outs1, lses1, state1 = _run(w, seed, 1, split)
    outs2, lses2, state2 = _run(w, seed, 2, split)
    for c in range(w.n_chunks):
        assert torch.equal(outs1[c].view(torch.int16), outs2[c].view(torch.int16)), (name, "out", c)
        assert torch.equal(lses1[c].view(torch.int32), lses2[c].view(torch.int32)), (name, "lse", c)
    for what, a, b in zip(("k_cache", "v_cache", "scores", "positions"), state1, state2):
        bits = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(a.view(bits), b.view(bits)), (name, what)
    # the run evicted: positions past the cache size are present
    assert int(state1[3].max()) >= w.cache_slots
