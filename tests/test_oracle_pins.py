"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test is chosen so that a plausible slip in the oracle (a dropped term,
a wrong sign or index, a transposed operand, an off-by-one in the causal
mask or in the recent window, a wrong GQA map, a reversed tie-break) fails at
least one of them:

* a hand-derived worked example with exact fractions (tests/golden);
* a pure-Python scalar brute force on tiny shapes (different structure);
* M >= L: the step must equal exact causal attention, computed here by
  torch's SDPA routine in fp64 on the whole sequence, and every slot's
  score must equal the full causal column mass of its key;
* W = M - S: eviction is forced onto the oldest tokens, i.e. sliding-window
  attention, computed by torch's SDPA with an explicit band mask;
* Q = 0: closed forms (harmonic sums) for the mass and uniform attention;
* mass conservation, slot-permutation invariance, batch independence,
  exact ties resolved to the lowest slot, the fill phase.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import h2o_oracle as orc
from oracle.brute import BruteState, brute_step

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _val(s: str) -> float:
    s = s.strip()
    if s.startswith("ln(") and s.endswith(")"):
        return math.log(float(Fraction(s[3:-1])))
    return float(Fraction(s))


def _rand_chunks(rng, B, Hq, Hkv, d, lens, qk=1.0):
    out = []
    for n in lens:
        out.append((rng.standard_normal((B, Hq, n, d)) * qk,
                    rng.standard_normal((B, Hkv, n, d)) * qk,
                    rng.standard_normal((B, Hkv, n, d))))
    return out


# ---------------------------------------------------------------- worked example
@pytest.mark.parametrize("run_idx", [0, 1])
def test_hand_worked_example(run_idx):
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    toks = g["tokens"]
    arr = lambda key, i: np.array([[[[_val(x) for x in toks[i][key]]]]])  # [1,1,1,d]
    scale = _val(g["scale"])
    M = g["cache_slots"]
    run = g["runs"][run_idx]
    W = run["W"]
    K, V, sig, pos = orc.empty_state(1, 1, M, 2)
    q01 = np.concatenate([arr("q", 0), arr("q", 1)], axis=2)
    k01 = np.concatenate([arr("k", 0), arr("k", 1)], axis=2)
    v01 = np.concatenate([arr("v", 0), arr("v", 1)], axis=2)
    st = orc.prefill(K, V, sig, pos, q01, k01, v01, W, scale)
    pe = g["prefill_expect"]
    np.testing.assert_allclose(st["out"][0, 0], [[_val(x) for x in r] for r in pe["out"]], atol=1e-14)
    np.testing.assert_allclose(st["lse"][0, 0], [_val(x) for x in pe["lse"]], atol=1e-14)
    np.testing.assert_allclose(st["sigma"][0, 0], [_val(x) for x in pe["sigma"]], atol=1e-14)
    assert st["pos"][0, 0].tolist() == pe["pos"]
    for s_idx, exp in enumerate(run["steps"]):
        t = 2 + s_idx
        st = orc.chunk_step(st["K"], st["V"], st["sigma"], st["pos"], st["T"],
                            arr("q", t), arr("k", t), arr("v", t), W, scale)
        np.testing.assert_allclose(st["out"][0, 0, 0], [_val(x) for x in exp["out"]], atol=1e-14)
        np.testing.assert_allclose(st["lse"][0, 0, 0], _val(exp["lse"]), atol=1e-14)
        np.testing.assert_allclose(st["delta_sigma"][0, 0], [_val(x) for x in exp["delta_sigma"]], atol=1e-14)
        np.testing.assert_allclose(st["mu"][0, 0, 0], _val(exp["mu"]), atol=1e-14)
        assert st["targets"][0, 0].tolist() == exp["targets"]
        np.testing.assert_allclose(st["sigma"][0, 0], [_val(x) for x in exp["sigma"]], atol=1e-14)
        assert st["pos"][0, 0].tolist() == exp["pos"]


# ---------------------------------------------------------------- brute force
def _to_lists(a):
    return a.tolist()


@pytest.mark.parametrize("N_C,M,W,steps", [(16, 16, 4, 6), (8, 16, 4, 6), (10, 16, 3, 5)])
def test_oracle_matches_brute_force(N_C, M, W, steps):
    rng = np.random.default_rng(1234 + N_C + M + W)
    B, Hq, Hkv, d, S = 2, 4, 2, 8, 4
    chunks = _rand_chunks(rng, B, Hq, Hkv, d, [N_C] + [S] * steps, qk=0.8)
    scale = 1.0 / math.sqrt(d)
    _, hist = orc.run_sequence(chunks, M, W, scale, keep_history=True)
    bs = BruteState(B, Hkv, M, d)
    for c, (q, k, v) in enumerate(chunks):
        out, lse, targets, mu = brute_step(bs, _to_lists(q), _to_lists(k), _to_lists(v), W, scale)
        st = hist[c]
        np.testing.assert_allclose(np.array(out), st["out"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(np.array(lse), st["lse"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(np.array(mu), st["mu"], rtol=0, atol=1e-12)
        assert np.array(targets).tolist() == st["targets"].tolist()
        np.testing.assert_allclose(np.array(bs.sigma), st["sigma"], rtol=0, atol=1e-12)
        assert np.array(bs.pos).tolist() == st["pos"].tolist()


def test_brute_force_and_oracle_agree_on_planted_ties():
    rng = np.random.default_rng(7)
    B, Hq, Hkv, d, M, S, W = 1, 2, 1, 4, 8, 3, 2
    K = rng.standard_normal((B, Hkv, M, d))
    V = rng.standard_normal((B, Hkv, M, d))
    pos = np.arange(M, dtype=np.int64)[None, None, :].copy()
    T = M
    # Q = 0 makes every visible key get the same mass, so the tie structure of
    # sigma is preserved: slots 1, 3, 4, 5 and 6 tie at the minimum.
    sig = np.array([[[5.0, 1.0, 2.0, 1.0, 1.0, 1.0, 1.0, 4.0]]])
    q = np.zeros((B, Hq, S, d))
    k = rng.standard_normal((B, Hkv, S, d))
    v = rng.standard_normal((B, Hkv, S, d))
    st = orc.chunk_step(K, V, sig, pos, T, q, k, v, W, 1.0)
    # candidates: pos < T - W = 6 -> slots 0..5; three evictions among the four
    # tied candidates {1, 3, 4, 5}: the lowest slots win (slot 6 is protected)
    assert st["targets"][0, 0].tolist() == [1, 3, 4]
    assert sorted(st["evicted"][0][0].tolist()) == [1, 3, 4]
    bs = BruteState(B, Hkv, M, d)
    bs.K, bs.V = K.tolist(), V.tolist()
    bs.sigma, bs.pos, bs.T = sig.tolist(), pos.tolist(), T
    _, _, targets, _ = brute_step(bs, q.tolist(), k.tolist(), v.tolist(), W, 1.0)
    assert targets[0][0] == [1, 3, 4]


# ---------------------------------------------------------------- M >= L: exact attention
def _torch_causal(qs, ks, vs, scale, mask=None):
    q = torch.from_numpy(qs)
    G = qs.shape[1] // ks.shape[1]
    k = torch.from_numpy(ks).repeat_interleave(G, dim=1)
    v = torch.from_numpy(vs).repeat_interleave(G, dim=1)
    if mask is None:
        out = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale)
        L = q.shape[2]
        mask = torch.ones(L, L, dtype=torch.bool).tril()
    else:
        mask = torch.from_numpy(mask)
        out = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    scores = (q @ k.transpose(-1, -2)) * scale
    scores = scores.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(scores, dim=-1)
    probs = torch.softmax(scores, dim=-1)
    return out.numpy(), lse.numpy(), probs.numpy()


@pytest.mark.parametrize("M", [64, 80])
def test_full_cache_equals_exact_causal_attention(M):
    rng = np.random.default_rng(99)
    B, Hq, Hkv, d = 2, 4, 2, 16
    lens = [24, 8, 8, 8, 16]        # L = 64 <= M
    chunks = _rand_chunks(rng, B, Hq, Hkv, d, lens)
    scale = 1.0 / math.sqrt(d)
    st, hist = orc.run_sequence(chunks, M, W=4, scale=scale, keep_history=True)
    qs = np.concatenate([c[0] for c in chunks], axis=2)
    ks = np.concatenate([c[1] for c in chunks], axis=2)
    vs = np.concatenate([c[2] for c in chunks], axis=2)
    out_ref, lse_ref, probs = _torch_causal(qs, ks, vs, scale)
    t0 = 0
    for c, n in enumerate(lens):
        np.testing.assert_allclose(hist[c]["out"], out_ref[:, :, t0:t0 + n], rtol=0, atol=1e-12)
        np.testing.assert_allclose(hist[c]["lse"], lse_ref[:, :, t0:t0 + n], rtol=0, atol=1e-12)
        t0 += n
    L = t0
    assert (st["pos"][:, :, :L] == np.arange(L)).all()
    assert (st["pos"][:, :, L:] == -1).all()
    # the score of key p is all the attention mass it received from the queries
    # p..L-1 of every head in its group
    G = Hq // Hkv
    colmass = probs.sum(axis=2).reshape(B, Hkv, G, L).sum(axis=2)
    np.testing.assert_allclose(st["sigma"][:, :, :L], colmass, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- W = M - S: sliding window
def test_window_m_minus_s_is_sliding_window_attention():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, d = 1, 4, 2, 8
    M, S, N_C = 24, 8, 12             # fill phase: 12 -> 20 -> 28 (first evicting step is partial)
    W = M - S
    lens = [N_C] + [S] * 7
    chunks = _rand_chunks(rng, B, Hq, Hkv, d, lens)
    scale = 1.0 / math.sqrt(d)
    _, hist = orc.run_sequence(chunks, M, W, scale, keep_history=True)
    qs = np.concatenate([c[0] for c in chunks], axis=2)
    ks = np.concatenate([c[1] for c in chunks], axis=2)
    vs = np.concatenate([c[2] for c in chunks], axis=2)
    L = qs.shape[2]
    mask = np.zeros((L, L), dtype=bool)
    t0 = 0
    for n in lens:
        for p in range(t0, t0 + n):
            mask[p, max(0, t0 - M):p + 1] = True
        t0 += n
    out_ref, lse_ref, _ = _torch_causal(qs, ks, vs, scale, mask=mask)
    t0 = 0
    for c, n in enumerate(lens):
        np.testing.assert_allclose(hist[c]["out"], out_ref[:, :, t0:t0 + n], rtol=0, atol=1e-12)
        np.testing.assert_allclose(hist[c]["lse"], lse_ref[:, :, t0:t0 + n], rtol=0, atol=1e-12)
        t0 += n
        T = t0
        kept = np.sort(hist[c]["pos"][0, 0])
        assert kept.tolist() == [-1] * max(0, M - T) + list(range(max(0, T - M), T))


# ---------------------------------------------------------------- Q = 0: closed forms
def test_zero_queries_closed_form():
    rng = np.random.default_rng(11)
    B, Hq, Hkv, d, M, S, N_C, W = 1, 6, 2, 4, 20, 5, 9, 2
    G = Hq // Hkv
    lens = [N_C] + [S] * 5
    chunks = [(np.zeros((B, Hq, n, d)), rng.standard_normal((B, Hkv, n, d)),
               rng.standard_normal((B, Hkv, n, d))) for n in lens]
    _, hist = orc.run_sequence(chunks, M, W, 1.0, keep_history=True)
    prev_pos = np.full((B, Hkv, M), -1)
    prev_K = np.zeros((B, Hkv, M, d))
    prev_V = np.zeros((B, Hkv, M, d))
    for c, n in enumerate(lens):
        st = hist[c]
        nv = int((prev_pos[0, 0] >= 0).sum())
        # every visible key of query i gets 1/(nv+i+1)
        inv = 1.0 / (nv + np.arange(n) + 1)
        exp_slot = G * inv.sum()
        exp_mu = G * np.array([inv[j:].sum() for j in range(n)])
        valid = prev_pos[0, 0] >= 0
        np.testing.assert_allclose(st["delta_sigma"][0, 0][valid], exp_slot, rtol=1e-13)
        assert (st["delta_sigma"][0, 0][~valid] == 0).all()
        np.testing.assert_allclose(st["mu"][0, 0], exp_mu, rtol=1e-13)
        np.testing.assert_allclose(st["lse"][0, 0], np.log(nv + np.arange(n) + 1), rtol=1e-13)
        q, k, v = chunks[c]
        for i in range(n):
            vis = np.concatenate([prev_V[0, 0][valid], v[0, 0, :i + 1]], axis=0)
            np.testing.assert_allclose(st["out"][0, 0, i], vis.mean(axis=0), atol=1e-13)
        prev_pos, prev_K, prev_V = st["pos"], st["K"], st["V"]


# ---------------------------------------------------------------- invariants
def test_mass_conservation_per_step():
    rng = np.random.default_rng(3)
    B, Hq, Hkv, d, M, S, N_C, W = 2, 8, 2, 16, 48, 16, 32, 8
    G = Hq // Hkv
    chunks = _rand_chunks(rng, B, Hq, Hkv, d, [N_C] + [S] * 6)
    _, hist = orc.run_sequence(chunks, M, W, keep_history=True)
    for c, st in enumerate(hist):
        n = N_C if c == 0 else S
        tot = st["delta_sigma"].sum(axis=-1) + st["mu"].sum(axis=-1)
        np.testing.assert_allclose(tot, n * G, rtol=1e-12)


def test_slot_permutation_invariance():
    rng = np.random.default_rng(21)
    B, Hq, Hkv, d, M, S, W = 1, 4, 2, 8, 32, 8, 4
    K = rng.standard_normal((B, Hkv, M, d))
    V = rng.standard_normal((B, Hkv, M, d))
    sig = rng.uniform(0.5, 3.0, (B, Hkv, M))
    pos = np.stack([rng.permutation(M) for _ in range(Hkv)])[None].astype(np.int64)
    T = M
    q = rng.standard_normal((B, Hq, S, d))
    k = rng.standard_normal((B, Hkv, S, d))
    v = rng.standard_normal((B, Hkv, S, d))
    a = orc.chunk_step(K, V, sig, pos, T, q, k, v, W)
    perm = rng.permutation(M)
    b = orc.chunk_step(K[:, :, perm], V[:, :, perm], sig[:, :, perm], pos[:, :, perm], T, q, k, v, W)
    np.testing.assert_allclose(a["out"], b["out"], atol=1e-12)
    np.testing.assert_allclose(a["lse"], b["lse"], atol=1e-12)
    np.testing.assert_allclose(a["delta_sigma"][:, :, perm], b["delta_sigma"], atol=1e-12)
    np.testing.assert_allclose(a["mu"], b["mu"], atol=1e-12)
    for h in range(Hkv):
        # the same tokens are evicted (scores are distinct, so no tie is involved)
        assert sorted(pos[0, h, a["evicted"][0][h]].tolist()) == \
            sorted(pos[0, h, perm][b["evicted"][0][h]].tolist())


def test_batch_elements_are_independent():
    rng = np.random.default_rng(8)
    B, Hq, Hkv, d, M, S, N_C, W = 3, 4, 2, 8, 24, 6, 18, 3
    chunks = _rand_chunks(rng, B, Hq, Hkv, d, [N_C] + [S] * 4)
    full = orc.run_sequence(chunks, M, W)
    for b in range(B):
        one = orc.run_sequence([(q[b:b + 1], k[b:b + 1], v[b:b + 1]) for q, k, v in chunks], M, W)
        np.testing.assert_allclose(full["sigma"][b:b + 1], one["sigma"], atol=1e-13)
        assert (full["pos"][b:b + 1] == one["pos"]).all()
        np.testing.assert_array_equal(full["K"][b:b + 1], one["K"])


def test_fill_phase_uses_free_slots_in_order():
    rng = np.random.default_rng(4)
    B, Hq, Hkv, d, M, S, N_C, W = 1, 2, 1, 4, 20, 6, 5, 2
    chunks = _rand_chunks(rng, B, Hq, Hkv, d, [N_C] + [S] * 4)
    _, hist = orc.run_sequence(chunks, M, W, keep_history=True)
    assert hist[0]["targets"][0, 0].tolist() == list(range(5))
    assert hist[1]["targets"][0, 0].tolist() == list(range(5, 11))
    assert hist[2]["targets"][0, 0].tolist() == list(range(11, 17))
    # 3 free slots left (17, 18, 19): they are used and 3 more are evicted
    t3 = hist[3]["targets"][0, 0].tolist()
    assert {17, 18, 19} <= set(t3) and len(hist[3]["evicted"][0][0]) == 3
    assert all(p >= 0 for p in hist[3]["pos"][0, 0])


def test_infeasible_eviction_raises():
    sig = np.zeros(4)
    pos = np.array([0, 1, 2, 3])
    with pytest.raises(ValueError):
        orc.select_targets(sig, pos, T=4, W=3, S=2)     # only slot 0 is evictable


# ---------------------------------------------------------------- backward
def _loss_and_out(K, V, pos, q, k, v, dO, scale):
    B, Hkv = K.shape[:2]
    G = q.shape[1] // Hkv
    outs = np.empty(q.shape)
    for b in range(B):
        for h in range(Hkv):
            o, _, _, _ = orc.attend_head(K[b, h], V[b, h], pos[b, h], q[b, h * G:(h + 1) * G],
                                         k[b, h], v[b, h], scale)
            outs[b, h * G:(h + 1) * G] = o
    return float((outs * dO).sum())


def _bwd_case(seed=17):
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, d, M, S = 1, 4, 2, 4, 6, 3
    K = rng.standard_normal((B, Hkv, M, d))
    V = rng.standard_normal((B, Hkv, M, d))
    pos = np.array([[[0, 3, -1, 1, 2, -1], [4, -1, 0, 1, 2, 3]]])
    q = rng.standard_normal((B, Hq, S, d))
    k = rng.standard_normal((B, Hkv, S, d))
    v = rng.standard_normal((B, Hkv, S, d))
    dO = rng.standard_normal((B, Hq, S, d))
    return K, V, pos, q, k, v, dO, 0.7


def test_backward_matches_central_differences():
    K, V, pos, q, k, v, dO, scale = _bwd_case()
    grads = orc.chunk_backward(K, V, pos, q, k, v, dO, scale)
    args = [K, V, q, k, v]
    names = ["K", "V", "q", "k", "v"]
    gmap = {"q": grads[0], "K": grads[1], "V": grads[2], "k": grads[3], "v": grads[4]}
    eps = 1e-6
    for ai, name in enumerate(names):
        x = args[ai]
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + eps
            lp = _loss_and_out(*_pack(args, pos), dO, scale)
            x[idx] = old - eps
            lm = _loss_and_out(*_pack(args, pos), dO, scale)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(gmap[name], num, rtol=1e-6, atol=1e-8, err_msg=name)
    # free slots get no gradient
    assert (gmap["K"][0, 0, [2, 5]] == 0).all() and (gmap["V"][0, 1, 1] == 0).all()


def _pack(args, pos):
    K, V, q, k, v = args
    return K, V, pos, q, k, v


def test_backward_matches_torch_autograd():
    K, V, pos, q, k, v, dO, scale = _bwd_case(23)
    grads = orc.chunk_backward(K, V, pos, q, k, v, dO, scale)
    B, Hkv, M, d = K.shape
    Hq, S = q.shape[1], q.shape[2]
    G = Hq // Hkv
    tK = torch.tensor(K, requires_grad=True)
    tV = torch.tensor(V, requires_grad=True)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    # textbook SDPA over [cache slots ++ chunk keys] with a fixed boolean mask
    keys = torch.cat([tK, tk], dim=2).repeat_interleave(G, dim=1)
    vals = torch.cat([tV, tv], dim=2).repeat_interleave(G, dim=1)
    mask = torch.zeros(B, Hq, S, M + S, dtype=torch.bool)
    for h in range(Hq):
        mask[0, h, :, :M] = torch.from_numpy(pos[0, h // G] >= 0)
        mask[0, h, :, M:] = torch.ones(S, S, dtype=torch.bool).tril()
    out = F.scaled_dot_product_attention(tq, keys, vals, attn_mask=mask, scale=scale)
    (out * torch.from_numpy(dO)).sum().backward()
    np.testing.assert_allclose(grads[0], tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(grads[1], tK.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(grads[2], tV.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(grads[3], tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(grads[4], tv.grad.numpy(), atol=1e-12)


# ---------------------------------------------------------------- gradient through the buffer
# oracle/recurrence_grad.py differentiates the whole row with the eviction
# decisions held fixed.  Pinned against: the step oracle's forward, the
# single-step textbook gradient, plain causal attention when nothing is
# evicted, and central differences with evictions.
from oracle import recurrence_grad as rg  # noqa: E402


def _row_case(seed, B, Hq, Hkv, d, lens, M, W):
    rng = np.random.default_rng(seed)
    chunks = _rand_chunks(rng, B, Hq, Hkv, d, lens)
    scale = 1.0 / math.sqrt(d)
    _, hist = orc.run_sequence(chunks, M, W=W, scale=scale, keep_history=True)
    targets = [h["targets"] for h in hist]
    d_outs = [rng.standard_normal(c[0].shape) for c in chunks]
    return chunks, targets, d_outs, hist, scale


def test_row_forward_matches_chunk_steps():
    chunks, targets, _, hist, scale = _row_case(31, 2, 4, 2, 8, [8, 4, 4, 4, 4, 4], M=12, W=2)
    assert any(len(e) for h in hist for per_b in h["evicted"] for e in per_b if e is not None)
    t = lambda x: torch.from_numpy(np.asarray(x, dtype=np.float64))
    outs = rg.row_forward([t(c[0]) for c in chunks], [t(c[1]) for c in chunks], [t(c[2]) for c in chunks],
                          targets, 12, scale)
    for c, o in enumerate(outs):
        np.testing.assert_allclose(o.numpy(), hist[c]["out"], rtol=0, atol=1e-12, err_msg=f"chunk {c}")


def test_row_grads_of_one_chunk_are_the_step_gradient():
    chunks, targets, d_outs, _, scale = _row_case(32, 1, 4, 2, 8, [7], M=10, W=2)
    (dq, dk, dv), = rg.row_grads(chunks, d_outs, targets, 10, scale)
    K, V, _, pos = orc.empty_state(1, 2, 10, 8)
    ref = orc.chunk_backward(K, V, pos, *chunks[0], d_outs[0], scale)
    np.testing.assert_allclose(dq, ref[0], atol=1e-12)
    np.testing.assert_allclose(dk, ref[3], atol=1e-12)
    np.testing.assert_allclose(dv, ref[4], atol=1e-12)


def test_row_grads_without_eviction_are_causal_attention_grads():
    lens = [10, 5, 5, 4]
    chunks, targets, d_outs, _, scale = _row_case(33, 1, 4, 2, 8, lens, M=32, W=3)
    grads = rg.row_grads(chunks, d_outs, targets, 32, scale)
    G = 2
    q = torch.tensor(np.concatenate([c[0] for c in chunks], axis=2), requires_grad=True)
    k = torch.tensor(np.concatenate([c[1] for c in chunks], axis=2), requires_grad=True)
    v = torch.tensor(np.concatenate([c[2] for c in chunks], axis=2), requires_grad=True)
    out = F.scaled_dot_product_attention(q, k.repeat_interleave(G, dim=1), v.repeat_interleave(G, dim=1),
                                         is_causal=True, scale=scale)
    (out * torch.from_numpy(np.concatenate(d_outs, axis=2))).sum().backward()
    t0 = 0
    for c, n in enumerate(lens):
        for got, ref in zip(grads[c], (q.grad, k.grad, v.grad)):
            np.testing.assert_allclose(got, ref.numpy()[:, :, t0:t0 + n], atol=1e-12, err_msg=f"chunk {c}")
        t0 += n


def test_row_grads_match_central_differences_with_evictions():
    M = 9
    chunks, targets, d_outs, hist, scale = _row_case(34, 1, 2, 1, 4, [6, 3, 3, 3], M=M, W=2)
    assert any(len(e) for h in hist[1:] for per_b in h["evicted"] for e in per_b if e is not None)
    grads = rg.row_grads(chunks, d_outs, targets, M, scale)

    def loss(ch):
        t = lambda x: torch.from_numpy(np.asarray(x, dtype=np.float64))
        outs = rg.row_forward([t(c[0]) for c in ch], [t(c[1]) for c in ch], [t(c[2]) for c in ch],
                              targets, M, scale)
        return sum(float((o * t(g)).sum()) for o, g in zip(outs, d_outs))

    rng = np.random.default_rng(35)
    eps = 1e-6
    work = [[np.array(x) for x in c] for c in chunks]
    for c in range(len(chunks)):
        for a in range(3):
            x = work[c][a]
            for _ in range(4):
                idx = tuple(int(rng.integers(0, s)) for s in x.shape)
                old = x[idx]
                x[idx] = old + eps
                lp = loss(work)
                x[idx] = old - eps
                lm = loss(work)
                x[idx] = old
                np.testing.assert_allclose(grads[c][a][idx], (lp - lm) / (2 * eps), rtol=1e-5, atol=1e-8,
                                           err_msg=f"chunk {c} tensor {a} index {idx}")


# ---------------------------------------------------------------- position policies
# "recent" keeps the newest tokens, "sink_recent" also the first n_sink: the
# cache is then a closed form of T, and attention is SDPA with the matching
# band mask over the whole sequence.
def _policy_mask(lens, M, n_sink):
    L = sum(lens)
    mask = np.zeros((L, L), dtype=bool)
    t0 = 0
    for n in lens:
        lo = t0 - (M - n_sink)              # oldest non-sink position held before the chunk
        for i in range(n):
            t = t0 + i
            p = np.arange(L)
            mask[t] = (p <= t) & ((p >= lo) | (p < n_sink) | (p >= t0))
        t0 += n
    return mask


@pytest.mark.parametrize("policy,n_sink", [("recent", 0), ("sink_recent", 3)])
def test_position_policies_are_banded_attention(policy, n_sink):
    rng = np.random.default_rng(41)
    B, Hq, Hkv, d = 1, 4, 2, 8
    M, W = 20, 4
    lens = [12, 6, 6, 6, 6, 6]
    chunks = _rand_chunks(rng, B, Hq, Hkv, d, lens)
    scale = 1.0 / math.sqrt(d)
    _, hist = orc.run_sequence(chunks, M, W=W, scale=scale, keep_history=True, policy=policy,
                               n_sink=n_sink)
    qs = np.concatenate([c[0] for c in chunks], axis=2)
    ks = np.concatenate([c[1] for c in chunks], axis=2)
    vs = np.concatenate([c[2] for c in chunks], axis=2)
    out_ref, lse_ref, _ = _torch_causal(qs, ks, vs, scale, mask=_policy_mask(lens, M, n_sink))
    t0 = 0
    for c, n in enumerate(lens):
        np.testing.assert_allclose(hist[c]["out"], out_ref[:, :, t0:t0 + n], rtol=0, atol=1e-12)
        np.testing.assert_allclose(hist[c]["lse"], lse_ref[:, :, t0:t0 + n], rtol=0, atol=1e-12)
        t0 += n
        held = np.sort(hist[c]["pos"][0, 0][hist[c]["pos"][0, 0] >= 0])
        keep = min(t0, M)
        expect = np.arange(t0 - keep, t0) if t0 <= M or n_sink == 0 else \
            np.concatenate([np.arange(n_sink), np.arange(t0 - (M - n_sink), t0)])
        np.testing.assert_array_equal(held, expect)
        assert (hist[c]["sigma"] == 0).all()          # no score is kept


def test_h2o_with_window_m_minus_s_equals_recent():
    rng = np.random.default_rng(42)
    B, Hq, Hkv, d = 1, 2, 1, 8
    M, S = 16, 4
    lens = [8] + [S] * 6
    chunks = _rand_chunks(rng, B, Hq, Hkv, d, lens)
    a = orc.run_sequence(chunks, M, W=M - S, keep_history=True)[1]
    b = orc.run_sequence(chunks, M, W=M - S, keep_history=True, policy="recent")[1]
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x["targets"], y["targets"])
        np.testing.assert_allclose(x["out"], y["out"], rtol=0, atol=0)
