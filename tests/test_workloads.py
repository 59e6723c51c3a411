"""Seeded input generators: determinism, heavy-hitter planting, bf16 rounding."""
import numpy as np
import torch

from kv_cache_eviction_amd import workloads as wl


def test_named_workloads_shapes():
    c2 = wl.WORKLOADS["llama8b_64k"]
    assert (c2.n_steps, c2.group, c2.n_chunks) == (62, 4, 63)
    c3 = wl.WORKLOADS["llama8b_128k"]
    assert c3.n_steps == 126 and (c3.cache_slots - c3.prefill) % c3.chunk == 0
    c4 = wl.WORKLOADS["decode_b32"]
    assert c4.n_steps == 256 and c4.chunk == 16 and c4.batch == 32
    c5 = wl.WORKLOADS["widegqa_128k"]
    assert c5.n_steps == 62 and c5.group == 8
    s128 = wl.WORKLOADS["llama8b_64k_s128"]
    assert (s128.n_steps, s128.chunk, s128.group) == (496, 128, 4)
    c1 = wl.WORKLOADS["tiny"]
    assert c1.n_steps == 12 and c1.dtype == "fp32"
    for w in wl.WORKLOADS.values():
        assert w.cache_slots - w.recent_window >= w.chunk      # every eviction is feasible
        assert w.prefill <= w.cache_slots


def test_generators_are_deterministic_and_seed_dependent():
    w = wl.workload("tiny")
    a = wl.chunk_inputs(w, 0, 3)
    b = wl.chunk_inputs(w, 0, 3)
    c = wl.chunk_inputs(w, 1, 3)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a[0], c[0])
    q, k, v = a
    assert q.shape == (1, 4, 64, 64) and k.shape == (1, 2, 64, 64) and q.dtype == np.float32


def test_heavy_hitter_planting():
    w = wl.workload("tiny")
    pos, u = wl.heavy_hitters(w, 0)
    assert pos.size == round(0.02 * w.total_len) and np.unique(pos).size == pos.size
    np.testing.assert_allclose(np.linalg.norm(u, axis=-1), 1.0, rtol=1e-6)
    # a planted key differs from an unplanted redraw by exactly 4u
    c = 1
    t0, n = w.chunk_bounds(c)
    hit = pos[(pos >= t0) & (pos < t0 + n)] - t0
    assert hit.size > 0
    _, k, _ = wl.chunk_inputs(w, 0, c)
    _, k0, _ = wl.chunk_inputs(w, 0, c, hh=(np.array([], dtype=np.int64), u))
    diff = (k - k0)[0][:, hit, :]
    np.testing.assert_allclose(diff, 4.0 * np.broadcast_to(u[0][:, None, :], diff.shape), atol=1e-5)


def test_zipf_positions_distinct_and_skewed():
    w = wl.workload("llama8b_128k")
    pos, _ = wl.heavy_hitters(w, 0)
    assert pos.size == round(0.005 * 131072) and np.unique(pos).size == pos.size
    # a Zipf(1.1) law puts most draws near the start of the sequence
    assert (pos < 1024).sum() > (pos >= 65536).sum()


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ours = wl.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = wl.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())
