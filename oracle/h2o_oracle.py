"""fp64 CPU oracle of the chunked H2O (heavy-hitter) attention step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or run anything under
``oracle/``.  The product path (``kv_cache_eviction_amd``) never does, and it
shares no code with this file: this is plain numpy written from the
definition, slow and obviously correct, so that a reader can check it
against the pages by eye.

Sources (cited by title, section and figure):

* "Learning how to Forget: Fine-tuning for Long-Context Sparse Attention"
  (arXiv 2608.19920), below "LHF".
  - Fig. 1(a): a row of chunks, a prefill chunk of length N_C followed by
    chunks of length S.
  - §1 Introduction ¶1: sparse attention keeps keys and values in a
    fixed-size KV cache whose slots are evicted once it is full.
  - §1 ¶3: grouped query attention: the query heads of one group share a KV
    head.
  - §1 ¶4 and the abstract: H2O, the heavy-hitter oracle (reference [72] of
    the paper), with an SDPA kernel that also returns summed attention
    weights (docshare page, FAQ answer on H2O).
  - contributions bullet of §1: the KV cache buffer follows a linear
    recurrence, each step overwriting some slots of the previous buffer.
* H2O: Heavy-Hitter Oracle (reference [72] of LHF): a slot's score is the
  attention mass its key has accumulated; the lowest-scoring slots go.

Readings where the pages are silent (each is listed in the design notes):

* score rule: plain cumulative sum of attention mass since insertion, summed
  over the chunk's queries and the query heads of the KV group;
* a newly written slot starts with the mass its key received from the
  chunk's own (causal) queries in the step that wrote it;
* order inside a step: attend to the pre-eviction cache, add the mass, then
  select victims, then overwrite;
* while free slots remain they are filled first, in ascending slot order;
  only the shortfall is evicted;
* protected recent window: slot m is protected when pos[m] >= T - W, with T
  the number of tokens seen before the chunk;
* victims: the n_e smallest candidates ordered by (score, slot index);
* the chunk's token j goes to the j-th smallest target slot;
* the position policies "recent" and "sink_recent" (the pages' lr and slr
  rows among their five KV cache policies, Tables 1 and 6; sinks after the
  attention-sinks paper in their reference list) rank the candidates by
  (position, slot) instead of (score, slot), so the oldest tokens go;
  "sink_recent" also protects positions below n_sink (a config value: the
  pages give no number).  They keep no score: the step adds no mass and a
  written slot's score is 0;
* softmax scale 1/sqrt(d) unless given, natural-log logsumexp, query head h
  uses KV head h // G; Q and K arrive with any positional encoding applied.

The state of one (batch, KV head) is K, V ``[M, d]``, scores ``sigma[M]``,
token positions ``pos[M]`` (-1 marks a free slot) and the shared count T of
tokens seen so far.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "POLICIES", "empty_state", "attend_head", "select_targets", "chunk_step", "prefill",
    "chunk_backward", "run_sequence",
]

POLICIES = ("h2o", "recent", "sink_recent")


def empty_state(B: int, Hkv: int, M: int, d: int):
    """An empty cache: zero K/V/scores and every slot free (pos = -1)."""
    K = np.zeros((B, Hkv, M, d))
    V = np.zeros((B, Hkv, M, d))
    sigma = np.zeros((B, Hkv, M))
    pos = np.full((B, Hkv, M), -1, dtype=np.int64)
    return K, V, sigma, pos


def _keys_of_step(Kc, Vc, pos, k_new, v_new):
    """Keys visible to a chunk: the filled slots (ascending) then the chunk's keys."""
    valid = np.flatnonzero(pos >= 0)
    Kx = np.concatenate([Kc[valid], k_new], axis=0)
    Vx = np.concatenate([Vc[valid], v_new], axis=0)
    return valid, Kx, Vx


def _visibility(n_valid: int, S: int) -> np.ndarray:
    """Query i sees every filled slot and the chunk keys j <= i (causal in the chunk)."""
    vis = np.ones((S, n_valid + S), dtype=bool)
    vis[:, n_valid:] = np.tril(np.ones((S, S), dtype=bool))
    return vis


def attend_head(Kc, Vc, pos, q, k_new, v_new, scale):
    """Attention of one KV group for one chunk (LHF §1 ¶1, §1 ¶3, FAQ on H2O).

    q ``[G, S, d]``: the chunk's queries for the G query heads of the group.
    Returns ``out [G,S,d]``, ``lse [G,S]`` (natural log), ``delta_sigma[M]``
    (mass each filled slot received, summed over heads and queries; zero for
    free slots) and ``mu[S]`` (mass each chunk key received from the chunk's
    queries i >= j, summed over heads).
    """
    G, S, _ = q.shape
    M = Kc.shape[0]
    valid, Kx, Vx = _keys_of_step(Kc, Vc, pos, k_new, v_new)
    nv = valid.size
    vis = _visibility(nv, S)
    out = np.empty_like(q)
    lse = np.empty((G, S))
    mass = np.zeros(nv + S)
    for g in range(G):
        z = scale * (q[g] @ Kx.T)
        z = np.where(vis, z, -np.inf)
        zmax = z.max(axis=1, keepdims=True)
        e = np.exp(z - zmax)
        l = e.sum(axis=1, keepdims=True)
        P = e / l
        lse[g] = (zmax + np.log(l))[:, 0]
        out[g] = P @ Vx
        mass += P.sum(axis=0)
    delta_sigma = np.zeros(M)
    delta_sigma[valid] = mass[:nv]
    return out, lse, delta_sigma, mass[nv:]


def select_targets(sigma, pos, T: int, W: int, S: int, policy: str = "h2o", n_sink: int = 0):
    """Slots a chunk of S tokens is written to (LHF §1 ¶1; H2O [72]).

    Free slots are used first (ascending); the remaining n_e = S - n_free
    targets are the n_e candidates with the smallest (score, slot), where a
    candidate is a filled slot outside the recent window (pos < T - W).
    Position policies rank by (position, slot) instead; "sink_recent" also
    excludes positions below n_sink from the candidates.

    Returns ``(targets, evicted, cut_gap)``: ``targets`` ascending (token j
    goes to ``targets[j]``), ``evicted`` in selection order, and the score
    gap between the first kept and the last evicted candidate (``inf`` when
    no candidate is kept or none is evicted).
    """
    free = np.flatnonzero(pos < 0)
    n_free = min(S, free.size)
    n_e = S - n_free
    if policy not in POLICIES:
        raise ValueError(f"unknown policy {policy}")
    floor = n_sink if policy == "sink_recent" else 0
    cand = np.flatnonzero((pos >= floor) & (pos < T - W))
    if cand.size < n_e:
        raise ValueError(f"only {cand.size} evictable slots for {n_e} evictions")
    rank_key = sigma if policy == "h2o" else pos
    order = np.lexsort((cand, rank_key[cand]))   # primary key: score or position; ties: slot
    ranked = cand[order]
    evicted = ranked[:n_e]
    if 0 < n_e < ranked.size:
        cut_gap = float(rank_key[ranked[n_e]] - rank_key[ranked[n_e - 1]])
    else:
        cut_gap = math.inf
    targets = np.sort(np.concatenate([free[:n_free], evicted]))
    return targets, evicted, cut_gap


def chunk_step(K, V, sigma, pos, T: int, q, k_new, v_new, W: int, scale=None, policy: str = "h2o",
               n_sink: int = 0):
    """One H2O chunk step on every (batch, KV head); inputs are not modified.

    Arrays: K, V ``[B,Hkv,M,d]``; sigma ``[B,Hkv,M]``; pos ``[B,Hkv,M]``;
    q ``[B,Hq,S,d]``; k_new, v_new ``[B,Hkv,S,d]``; T = tokens seen before
    the chunk.  Steps, in order: attend (pre-eviction cache plus the chunk,
    causal in the chunk), add the step's mass to the filled slots' scores,
    select the targets, write the chunk's K/V, score and position into them.
    Returns a dict with the new state and the step's outputs.
    """
    B, Hkv, M, d = K.shape
    Hq, S = q.shape[1], q.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    K, V, sigma, pos = K.copy(), V.copy(), sigma.copy(), pos.copy()
    out = np.empty(q.shape)
    lse = np.empty((B, Hq, S))
    delta_sigma = np.zeros((B, Hkv, M))
    mu = np.zeros((B, Hkv, S))
    targets = np.zeros((B, Hkv, S), dtype=np.int64)
    evicted = [[None] * Hkv for _ in range(B)]
    cut_gap = np.full((B, Hkv), math.inf)
    for b in range(B):
        for h in range(Hkv):
            hs = slice(h * G, (h + 1) * G)
            o, ls, ds, m = attend_head(K[b, h], V[b, h], pos[b, h], q[b, hs],
                                       k_new[b, h], v_new[b, h], scale)
            out[b, hs], lse[b, hs] = o, ls
            if policy != "h2o":             # position policies keep no score
                ds, m = np.zeros_like(ds), np.zeros_like(m)
            delta_sigma[b, h], mu[b, h] = ds, m
            sig = sigma[b, h] + ds          # free slots stay 0 (ds is 0 there)
            R, E, gap = select_targets(sig, pos[b, h], T, W, S, policy, n_sink)
            sig[R] = m
            K[b, h, R] = k_new[b, h]
            V[b, h, R] = v_new[b, h]
            pos[b, h, R] = T + np.arange(S)
            sigma[b, h] = sig
            targets[b, h], evicted[b][h], cut_gap[b, h] = R, E, gap
    return dict(K=K, V=V, sigma=sigma, pos=pos, T=T + S, out=out, lse=lse,
                delta_sigma=delta_sigma, mu=mu, targets=targets,
                evicted=evicted, cut_gap=cut_gap)


def prefill(K, V, sigma, pos, q, k, v, W: int, scale=None, policy: str = "h2o", n_sink: int = 0):
    """The prefill chunk of length N_C (LHF Fig. 1(a)) into an empty cache."""
    if np.any(pos >= 0):
        raise ValueError("prefill expects an empty cache")
    if q.shape[2] > K.shape[2]:
        raise ValueError("prefill chunk longer than the cache")
    return chunk_step(K, V, sigma, pos, 0, q, k, v, W, scale, policy, n_sink)


def chunk_backward(K, V, pos, q, k_new, v_new, d_out, scale=None):
    """Gradient of one chunk's attention output with the eviction held fixed.

    The cache (K, V, pos) is the state before the step; the visible sets are
    those of ``attend_head`` and the scores are not differentiated.  Textbook
    softmax-attention gradient, per query head h with KV head h // G:
    dP = dO V_x^T, D_i = sum_x P_ix dP_ix, dZ = P * (dP - D), dq = scale dZ K_x,
    dK_x += scale dZ^T q, dV_x += P^T dO.
    Returns dq ``[B,Hq,S,d]``, dK and dV ``[B,Hkv,M,d]`` (zero at free
    slots), dk_new and dv_new ``[B,Hkv,S,d]``.
    """
    B, Hkv, M, d = K.shape
    Hq, S = q.shape[1], q.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = np.zeros(q.shape)
    dK = np.zeros(K.shape)
    dV = np.zeros(V.shape)
    dk_new = np.zeros(k_new.shape)
    dv_new = np.zeros(v_new.shape)
    for b in range(B):
        for h in range(Hkv):
            valid, Kx, Vx = _keys_of_step(K[b, h], V[b, h], pos[b, h], k_new[b, h], v_new[b, h])
            nv = valid.size
            vis = _visibility(nv, S)
            dKx = np.zeros_like(Kx)
            dVx = np.zeros_like(Vx)
            for g in range(G):
                hq = h * G + g
                z = np.where(vis, scale * (q[b, hq] @ Kx.T), -np.inf)
                e = np.exp(z - z.max(axis=1, keepdims=True))
                P = e / e.sum(axis=1, keepdims=True)
                dP = d_out[b, hq] @ Vx.T
                D = (P * dP).sum(axis=1, keepdims=True)
                dZ = P * (dP - D)
                dq[b, hq] = scale * (dZ @ Kx)
                dKx += scale * (dZ.T @ q[b, hq])
                dVx += P.T @ d_out[b, hq]
            dK[b, h, valid] = dKx[:nv]
            dV[b, h, valid] = dVx[:nv]
            dk_new[b, h] = dKx[nv:]
            dv_new[b, h] = dVx[nv:]
    return dq, dK, dV, dk_new, dv_new


def run_sequence(chunks, M: int, W: int, scale=None, keep_history: bool = False, policy: str = "h2o",
                 n_sink: int = 0):
    """Free-running H2O over a row of chunks ``[(q, k, v), ...]`` (prefill first).

    Returns the final state dict; with ``keep_history`` also the list of all
    per-step dicts.
    """
    q0, k0, _ = chunks[0]
    B, Hkv, _, d = k0.shape
    K, V, sigma, pos = empty_state(B, Hkv, M, d)
    hist = []
    st = prefill(K, V, sigma, pos, *chunks[0], W, scale, policy, n_sink)
    hist.append(st)
    for q, k, v in chunks[1:]:
        st = chunk_step(st["K"], st["V"], st["sigma"], st["pos"], st["T"], q, k, v, W, scale, policy, n_sink)
        hist.append(st)
    return (st, hist) if keep_history else st
