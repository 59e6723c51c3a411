"""Host logic of bench.py (no GPU): the single-GPU refusal, the algorithmic
work it divides by (visible pairs, flops, attention bytes, each against a
brute-force count over the same shapes), the rule for which chunk steps run
the fused short-chunk kernel, and the source-digest check of recorded HBM
traffic."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from kv_cache_eviction_amd import workloads as wl  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name,overrides", [
    ("tiny", {}),
    ("llama8b_64k", dict(total_len=2048 + 3 * 1024, cache_slots=2048)),
    ("decode_b32", dict(total_len=2048 + 5 * 16)),
])
def test_visible_pairs_and_flops_match_a_brute_count(name, overrides):
    w = wl.workload(name, **overrides)
    T = 0
    fl = bench.algorithmic_flops(w, backward=True, prefill_backward=True)
    fwd = [f for kind, f in fl if kind != "backward"]
    bwd = [f for kind, f in fl if kind == "backward"]
    assert len(fwd) == w.n_chunks and len(bwd) == w.n_chunks
    for c in range(w.n_chunks):
        _, n = w.chunk_bounds(c)
        filled = min(T, w.cache_slots)           # slots that hold a token when chunk c arrives
        pairs = sum(filled + (i + 1) for i in range(n))   # query i sees the cache and chunk keys 0..i
        assert bench.visible_pairs(w, c, T) == pairs
        assert fwd[c] == 4.0 * w.batch * w.n_q_heads * w.head_dim * pairs
        assert bwd[c] == 10.0 * w.batch * w.n_q_heads * w.head_dim * pairs
        T += n


def test_attention_bytes_count_each_tensor_once():
    w = wl.workload("decode_b32", total_len=2048 + 4 * 16)
    T = 0
    for c in range(w.n_chunks):
        _, n = w.chunk_bounds(c)
        mv = min(T, w.cache_slots)
        e, B, Hq, Hkv, d = 2, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
        q = o = B * Hq * n * d * e
        k_cache = v_cache = B * Hkv * mv * d * e
        k_new = v_new = B * Hkv * n * d * e
        lse = B * Hq * n * 4
        assert bench.attn_bytes(w, c, T) == q + o + k_cache + v_cache + k_new + v_new + lse
        T += n


@pytest.mark.parametrize("name,overrides,policy,expected", [
    ("decode_b32", {}, "h2o", True),
    ("llama8b_64k_s128", {}, "h2o", True),                 # G*S = 512 rows, 64 + 4 key blocks
    ("llama8b_64k", {}, "h2o", False),                     # G*S = 4096 rows
    ("decode_b32", {}, "recent", False),                   # position policies need no masses
    ("decode_b32", dict(head_dim=64, n_q_heads=4, n_kv_heads=1, cache_slots=2272), "h2o", True),
    ("decode_b32", dict(head_dim=64, n_q_heads=4, n_kv_heads=1, cache_slots=2273), "h2o", False),
    ("tiny", dict(chunk=16), "h2o", False),                # fp32
])
def test_fused_kernel_rule(name, overrides, policy, expected):
    """The library takes a step into the fused kernel for bf16, d 64 or 128,
    at most 512 query rows per KV group and at most 72 key blocks of 32; the
    last two cases of the cache limit are the GPU tests' shapes on either side
    of it."""
    w = wl.workload(name, **overrides)
    assert bench.takes_fused_kernel(w, policy) is expected


def test_recorded_traffic_requires_the_counted_source(tmp_path, monkeypatch):
    digest = bench.source_digest(bench.ATTN_SOURCES)
    f = tmp_path / "hbm.md"
    f.write_text("| kernel | workload | bytes | digest |\n|---|---|---|---|\n"
                 f"| attn_fwd_bf16_kernel | llama8b_64k | 123456 | {digest} |\n"
                 "| attn_fwd_bf16_kernel | llama8b_128k | 654321 | 0123456789abcdef |\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.recorded_traffic("attn_fwd_bf16_kernel", "llama8b_64k") == 123456
    assert bench.recorded_traffic("attn_fwd_bf16_kernel", "llama8b_128k") is None    # other source
    assert bench.recorded_traffic("attn_fwd_bf16_kernel", "decode_b32") is None      # not recorded


@pytest.mark.parametrize("batch,heads,n,expect", [
    (32, 8, 1, ("batch", 32)),
    (32, 8, 2, ("batch", 16)),
    (32, 8, 4, ("batch", 8)),
    (32, 8, 3, None),              # 32 sequences do not split 3 ways
    (1, 8, 2, ("heads", 4)),       # one sequence: its KV heads split
    (1, 8, 8, ("heads", 1)),
    (1, 8, 3, None),
    (2, 8, 4, None),               # B > 1 splits the batch only
    (4, 8, 0, None),
])
def test_stream_groups_partition_the_pairs(batch, heads, n, expect):
    assert bench.plan_groups(batch, heads, n) == expect
    if expect is not None:
        kind, per = expect
        # the groups cover every (sequence, KV head) pair once
        total = per * n * (heads if kind == "batch" else batch) if n > 1 else batch * heads
        assert total == batch * heads


def test_streams_refuse_workloads_with_a_backward():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "widegqa_128k",
                        "--streams", "2"], capture_output=True, text=True, timeout=300,
                       env={**os.environ, "HIP_VISIBLE_DEVICES": ""})
    assert r.returncode == 2
    assert "forward-only" in r.stderr


def test_state_bytes_count_each_state_tensor_once():
    w = wl.workload("decode_b32", total_len=2048 + 3 * 16)
    for c in range(1, w.n_chunks):
        _, n = w.chunk_bounds(c)
        per_head = (w.cache_slots * 4          # scores read
                    + w.cache_slots * 4        # scores written back
                    + w.cache_slots * 4        # positions read
                    + n * 4                    # the chunk's positions written
                    + 2 * n * w.head_dim * 2)  # its K and V rows written (bf16)
        assert bench.state_bytes(w, c) == w.batch * w.n_kv_heads * per_head
