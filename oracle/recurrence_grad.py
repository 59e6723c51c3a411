"""fp64 CPU oracle of the gradient through the KV buffer over a row of chunks.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or run anything under
``oracle/``; the product path never does and shares no code with it.

Source: "Learning how to Forget: Fine-tuning for Long-Context Sparse
Attention" (arXiv 2608.19920), Fig. 1(b): training unrolls the row of chunks
and back-propagates through the buffer; the contributions bullet of §1: the
buffer follows a linear recurrence, each step overwriting some slots of the
previous buffer with the chunk's keys and values.

Reading (the same frozen-eviction reading as ``h2o_oracle.chunk_backward``
for one step): the eviction decisions of the forward run -- which slot each
chunk token went to -- are held fixed, and the scores are not
differentiated.  The whole row is then a differentiable function of every
chunk's q, k and v.  This module writes that function out step by step in
torch fp64 (attend to the filled slots plus the chunk's keys j <= i, then
copy the chunk's rows into their slots) and lets autograd differentiate
sum_c <out_c, dO_c>.  Pins (tests/test_oracle_pins.py): central finite
differences, the single-chunk case against ``h2o_oracle.chunk_backward``, the
forward against ``h2o_oracle.chunk_step``, and the no-eviction case against
plain causal attention over the concatenated sequence.
"""
from __future__ import annotations

import math

import numpy as np
import torch

__all__ = ["row_forward", "row_grads"]


def row_forward(qs, ks, vs, targets, M: int, scale: float):
    """Outputs of every step of the row, as torch fp64 tensors.

    qs[c] ``[B,Hq,S_c,d]``, ks[c], vs[c] ``[B,Hkv,S_c,d]`` (torch, fp64);
    targets[c] ``[B,Hkv,S_c]``: the slot chunk c's token j is written to.
    The cache starts empty (every slot free).
    """
    B, Hkv, _, d = ks[0].shape
    Hq = qs[0].shape[1]
    G = Hq // Hkv
    K = torch.zeros(B, Hkv, M, d, dtype=torch.float64)
    V = torch.zeros_like(K)
    filled = torch.zeros(B, Hkv, M, dtype=torch.bool)
    outs = []
    for q, k, v, tg in zip(qs, ks, vs, targets):
        S = q.shape[2]
        per_b = []
        for b in range(B):
            per_h = []
            for hq in range(Hq):
                h = hq // G
                nv = int(filled[b, h].sum())
                keys = torch.cat([K[b, h][filled[b, h]], k[b, h]])
                vals = torch.cat([V[b, h][filled[b, h]], v[b, h]])
                visible = torch.ones(S, nv + S, dtype=torch.bool)
                visible[:, nv:] = torch.tril(torch.ones(S, S, dtype=torch.bool))
                z = (scale * (q[b, hq] @ keys.T)).masked_fill(~visible, -math.inf)
                per_h.append(torch.softmax(z, dim=-1) @ vals)
            per_b.append(torch.stack(per_h))
        outs.append(torch.stack(per_b))
        # the step's writes: a new buffer equal to the old one except the targets
        K, V, filled = K.clone(), V.clone(), filled.clone()
        for b in range(B):
            for h in range(Hkv):
                idx = torch.as_tensor(np.asarray(tg[b, h]), dtype=torch.long)
                K[b, h, idx] = k[b, h]
                V[b, h, idx] = v[b, h]
                filled[b, h, idx] = True
    return outs


def row_grads(chunks, d_outs, targets, M: int, scale=None):
    """Gradients of sum_c <out_c, dO_c> with respect to every chunk's q, k, v.

    chunks[c] = (q, k, v) fp64 numpy arrays; d_outs[c] like q; targets[c]
    ``[B,Hkv,S_c]`` slot indices (held fixed).  Returns a list of
    (dq, dk, dv) numpy arrays, one per chunk.
    """
    d = chunks[0][0].shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    params = [tuple(torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True) for x in ch)
              for ch in chunks]
    outs = row_forward([p[0] for p in params], [p[1] for p in params], [p[2] for p in params],
                       targets, M, scale)
    loss = sum((o * torch.tensor(np.asarray(g, dtype=np.float64))).sum() for o, g in zip(outs, d_outs))
    loss.backward()
    return [tuple(t.grad.numpy().copy() for t in p) for p in params]
