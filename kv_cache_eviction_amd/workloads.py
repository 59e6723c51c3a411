"""Seeded synthetic workloads for the chunked H2O attention step.

This module only draws inputs. It holds none of the method's arithmetic, so
both the fp64 oracle (``oracle/``) and the HIP path can consume what it
produces without sharing any code of the step itself.

Shapes follow the chunk lattice of "Learning how to Forget: Fine-tuning for
Long-Context Sparse Attention" (arXiv 2608.19920), Fig. 1(a): a row starts
with a prefill chunk of length ``N_C`` and continues with chunks of length
``S``.  The 64k / 128k context lengths and the 2k / 1k chunk sizes mirror the
Helmet datasets and chunk sizes of its Tables 1-7; the pages' own data and
model weights are not used: every value below is synthetic.

Recipe (identical for every workload):

* chunk ``c`` (``c = 0`` is the prefill chunk) draws Q, K, V from
  ``numpy.random.default_rng([seed, cfg_id, c])`` as float32 standard
  normals, scaled by ``qk_std`` (Q and K) and ``v_std`` (V);
* heavy-hitter keys: ``round(hh_frac * L)`` distinct token positions get
  ``+4 u`` added to their key, with ``u`` a unit vector drawn once per
  (batch, KV head); positions are uniform without replacement, or drawn from
  a Zipf law over the sequence (rank r has probability proportional to
  ``r ** -zipf_a``, position r-1, duplicates redrawn); positions and ``u``
  come from ``default_rng([seed, cfg_id, 2**31 - 1])``;
* bf16 workloads round the float32 values to bf16 once (round to nearest
  even); both sides see exactly those stored values;
* the upstream gradient of the backward workload comes from
  ``default_rng([seed, cfg_id, c, 7])``, standard normal.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "heavy_hitters", "chunk_inputs",
    "chunk_grad_out", "to_bf16_bits", "bf16_bits_to_f32", "stored_to_f64",
]


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str            # "bf16" or "fp32": storage and MFMA input type
    prefill: int          # N_C
    chunk: int            # S
    total_len: int        # L (prefill + n_steps * S)
    cache_slots: int      # M
    recent_window: int    # W
    hh_frac: float
    hh_mode: str = "uniform"   # "uniform" | "zipf"
    qk_std: float = 1.0
    v_std: float = 1.0
    zipf_a: float = 1.1
    backward: bool = False
    note: str = field(default="", compare=False)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_steps(self) -> int:
        return (self.total_len - self.prefill) // self.chunk

    @property
    def n_chunks(self) -> int:
        return 1 + self.n_steps

    def chunk_bounds(self, c: int) -> tuple[int, int]:
        """(first token position, length) of chunk ``c``; chunk 0 is the prefill."""
        if c == 0:
            return 0, self.prefill
        return self.prefill + (c - 1) * self.chunk, self.chunk

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


_D = 128
WORKLOADS: dict[str, Workload] = {
    "tiny": Workload(
        "tiny", 1, batch=1, n_q_heads=4, n_kv_heads=2, head_dim=64, dtype="fp32",
        prefill=256, chunk=64, total_len=1024, cache_slots=256, recent_window=32,
        hh_frac=0.02, note="tiny fp32 case, every step evicts"),
    "llama8b_64k": Workload(
        "llama8b_64k", 2, batch=1, n_q_heads=32, n_kv_heads=8, head_dim=_D, dtype="bf16",
        prefill=2048, chunk=1024, total_len=65536, cache_slots=2048, recent_window=256,
        hh_frac=0.01, qk_std=1.0 / math.sqrt(_D),
        note="Llama-3-8B-shaped attention layer, 64k context"),
    "llama8b_128k": Workload(
        "llama8b_128k", 3, batch=1, n_q_heads=32, n_kv_heads=8, head_dim=_D, dtype="bf16",
        prefill=2048, chunk=1024, total_len=131072, cache_slots=4096, recent_window=512,
        hh_frac=0.005, hh_mode="zipf", qk_std=1.0 / math.sqrt(_D),
        note="same shape, 128k context, Zipf-placed heavy hitters"),
    "decode_b32": Workload(
        "decode_b32", 4, batch=32, n_q_heads=32, n_kv_heads=8, head_dim=_D, dtype="bf16",
        prefill=2048, chunk=16, total_len=2048 + 256 * 16, cache_slots=2048,
        recent_window=256, hh_frac=0.01,
        note="decode-like small chunks, 32 sequences, bandwidth-bound"),
    "llama8b_64k_s128": Workload(
        "llama8b_64k_s128", 6, batch=1, n_q_heads=32, n_kv_heads=8, head_dim=_D, dtype="bf16",
        prefill=2048, chunk=128, total_len=65536, cache_slots=2048, recent_window=256,
        hh_frac=0.01, qk_std=1.0 / math.sqrt(_D),
        note="the 64k workload with 128-token chunks (the pages' S = 128 rows)"),
    "widegqa_128k": Workload(
        "widegqa_128k", 5, batch=1, n_q_heads=64, n_kv_heads=8, head_dim=_D, dtype="bf16",
        prefill=4096, chunk=2048, total_len=131072, cache_slots=8192, recent_window=512,
        hh_frac=0.01, backward=True,
        note="wide GQA (G=8), long chunks, forward and frozen-eviction backward"),
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields replaced (for small test variants)."""
    w = WORKLOADS[name]
    if overrides:
        d = {f: getattr(w, f) for f in w.__dataclass_fields__}
        d.update(overrides)
        w = Workload(**d)
    return w


def heavy_hitters(w: Workload, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Sorted heavy-hitter token positions and unit directions ``u[B, Hkv, d]``."""
    rng = np.random.default_rng([seed, w.cfg_id, 2**31 - 1])
    L = w.total_len
    n_hh = int(round(w.hh_frac * L))
    if w.hh_mode == "uniform":
        pos = rng.choice(L, size=n_hh, replace=False)
    elif w.hh_mode == "zipf":
        ranks = np.arange(1, L + 1, dtype=np.float64)
        p = ranks ** (-w.zipf_a)
        p /= p.sum()
        chosen: list[int] = []
        seen: set[int] = set()
        while len(chosen) < n_hh:
            for r in rng.choice(L, size=4 * n_hh, p=p):
                r = int(r)
                if r not in seen:
                    seen.add(r)
                    chosen.append(r)
                    if len(chosen) == n_hh:
                        break
        pos = np.asarray(chosen, dtype=np.int64)
    else:
        raise ValueError(f"unknown heavy-hitter mode {w.hh_mode!r}")
    u = rng.standard_normal((w.batch, w.n_kv_heads, w.head_dim))
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    return np.sort(pos.astype(np.int64)), u.astype(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def stored_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact float64 values of stored inputs (bf16 bit patterns or float32)."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def chunk_inputs(w: Workload, seed: int, c: int, hh=None):
    """Q ``[B,Hq,n,d]``, K and V ``[B,Hkv,n,d]`` of chunk ``c`` as stored values.

    bf16 workloads return uint16 bit patterns, fp32 workloads float32 arrays.
    ``hh`` may pass a precomputed ``heavy_hitters(w, seed)`` to save time.
    """
    t0, n = w.chunk_bounds(c)
    rng = np.random.default_rng([seed, w.cfg_id, c])
    B, Hq, Hkv, d = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    q = rng.standard_normal((B, Hq, n, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, n, d), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, n, d), dtype=np.float32)
    if w.qk_std != 1.0:
        q *= np.float32(w.qk_std)
        k *= np.float32(w.qk_std)
    if w.v_std != 1.0:
        v *= np.float32(w.v_std)
    pos, u = hh if hh is not None else heavy_hitters(w, seed)
    sel = pos[(pos >= t0) & (pos < t0 + n)] - t0
    if sel.size:
        k[:, :, sel, :] += np.float32(4.0) * u[:, :, None, :]
    if w.dtype == "bf16":
        return to_bf16_bits(q), to_bf16_bits(k), to_bf16_bits(v)
    return q, k, v


def chunk_grad_out(w: Workload, seed: int, c: int) -> np.ndarray:
    """Upstream gradient dO ``[B,Hq,n,d]`` for chunk ``c`` as stored values."""
    _, n = w.chunk_bounds(c)
    rng = np.random.default_rng([seed, w.cfg_id, c, 7])
    g = rng.standard_normal((w.batch, w.n_q_heads, n, w.head_dim), dtype=np.float32)
    return to_bf16_bits(g) if w.dtype == "bf16" else g
