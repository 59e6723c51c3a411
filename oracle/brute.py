"""Pure-Python scalar brute force of the H2O chunk step, for tiny inputs.

TEST INFRASTRUCTURE ONLY (same rule as ``h2o_oracle``).  It re-derives the
step with scalar loops, ``math.exp`` and correctly rounded ``math.fsum``
sums, and picks victims by repeated minimum scans instead of a sort, so that
it shares no structure with the numpy oracle it cross-checks.

The step follows "Learning how to Forget: Fine-tuning for Long-Context
Sparse Attention" (arXiv 2608.19920): Fig. 1(a) for the chunk lattice, §1
Introduction ¶1 for the fixed-size cache evicted once full, §1 ¶3 for
grouped query attention and the H2O heavy-hitter score of §1 ¶4, with the
same readings as the numpy oracle (scores summed over the chunk's queries
and the group's heads, pre-eviction attention, free slots first, recent
window pos >= T - W protected, ties to the lowest slot).

State layout: nested lists indexed ``[b][h][slot]`` (rows are lists of d
floats), positions -1 for free slots.
"""
from __future__ import annotations

import math

__all__ = ["BruteState", "brute_step"]


class BruteState:
    def __init__(self, B, Hkv, M, d):
        self.K = [[[[0.0] * d for _ in range(M)] for _ in range(Hkv)] for _ in range(B)]
        self.V = [[[[0.0] * d for _ in range(M)] for _ in range(Hkv)] for _ in range(B)]
        self.sigma = [[[0.0] * M for _ in range(Hkv)] for _ in range(B)]
        self.pos = [[[-1] * M for _ in range(Hkv)] for _ in range(B)]
        self.T = 0


def _dot(a, b):
    return math.fsum(x * y for x, y in zip(a, b))


def brute_step(st: BruteState, q, k_new, v_new, W: int, scale: float):
    """One chunk step in place; q[b][hq][i] rows, k_new/v_new[b][h][j] rows.

    Returns (out[b][hq][i][e], lse[b][hq][i], targets[b][h] list, mu[b][h]).
    """
    B = len(q)
    Hq = len(q[0])
    Hkv = len(k_new[0])
    G = Hq // Hkv
    S = len(k_new[0][0])
    M = len(st.pos[0][0])
    d = len(k_new[0][0][0])
    T = st.T
    out = [[None] * Hq for _ in range(B)]
    lse = [[None] * Hq for _ in range(B)]
    targets = [[None] * Hkv for _ in range(B)]
    mus = [[None] * Hkv for _ in range(B)]
    for b in range(B):
        for h in range(Hkv):
            pos = st.pos[b][h]
            slot_gain = [[] for _ in range(M)]
            chunk_gain = [[] for _ in range(S)]
            for g in range(G):
                hq = h * G + g
                out[b][hq] = []
                lse[b][hq] = []
                for i in range(S):
                    qi = q[b][hq][i]
                    # visible keys: every filled slot, then chunk keys 0..i
                    keys = [("slot", m) for m in range(M) if pos[m] >= 0]
                    keys += [("new", j) for j in range(i + 1)]
                    zs = []
                    for kind, x in keys:
                        krow = st.K[b][h][x] if kind == "slot" else k_new[b][h][x]
                        zs.append(scale * _dot(qi, krow))
                    zmax = max(zs)
                    es = [math.exp(z - zmax) for z in zs]
                    l = math.fsum(es)
                    lse[b][hq].append(zmax + math.log(l))
                    probs = [e / l for e in es]
                    o = []
                    for e_idx in range(d):
                        terms = []
                        for p, (kind, x) in zip(probs, keys):
                            vrow = st.V[b][h][x] if kind == "slot" else v_new[b][h][x]
                            terms.append(p * vrow[e_idx])
                        o.append(math.fsum(terms))
                    out[b][hq].append(o)
                    for p, (kind, x) in zip(probs, keys):
                        (slot_gain[x] if kind == "slot" else chunk_gain[x]).append(p)
            # score update
            sig = st.sigma[b][h]
            for m in range(M):
                if pos[m] >= 0:
                    sig[m] = math.fsum([sig[m]] + slot_gain[m])
            mu = [math.fsum(chunk_gain[j]) for j in range(S)]
            # targets: lowest free slots first, then repeated minimum scans
            chosen = []
            for m in range(M):
                if pos[m] < 0 and len(chosen) < S:
                    chosen.append(m)
            taken = set(chosen)
            while len(chosen) < S:
                best = None
                for m in range(M):
                    if m in taken or pos[m] < 0 or pos[m] >= T - W:
                        continue
                    if best is None or sig[m] < sig[best]:
                        best = m          # strict '<' keeps the lowest slot on ties
                if best is None:
                    raise ValueError("no evictable slot left")
                chosen.append(best)
                taken.add(best)
            R = sorted(chosen)
            for j, m in enumerate(R):
                st.K[b][h][m] = list(k_new[b][h][j])
                st.V[b][h][m] = list(v_new[b][h][j])
                sig[m] = mu[j]
                pos[m] = T + j
            targets[b][h] = R
            mus[b][h] = mu
    st.T = T + S
    return out, lse, targets, mus
