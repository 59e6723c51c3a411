"""The select kernel's parts: for chunks of 257..4096 tokens a KV head's
selection runs in several workgroups that each compute it in full and copy
a share of the chunk's rows; part 0 rewrites the head's scores and positions
only once every other part has counted its reads of them on a per-head
counter.  The wait is bounded and flags bit 1 of the device status word when
it gives up.  Parity of the parts' results with the oracle is covered by the
parity suites (every chunk longer than 256 tokens there runs several parts);
this file checks the handshake itself: normal steps never reach the bound,
and a wait that cannot be satisfied (an expected count raised by one, a
bound of a few polls, both through the test-only environment knobs read at
h2o_cache_init) ends and sets the flag instead of hanging.
"""
from __future__ import annotations

import pytest
import torch

from tests.parity_helpers import h2o_mod

pytestmark = pytest.mark.gpu


def _steps(h2o, cfg, n_steps, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    B, Hq, Hkv, d = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    cache = h2o.H2OCache(cfg)

    def rnd(*shape):
        return (torch.randn(*shape, generator=g) / d ** 0.25).to(torch.bfloat16).cuda()

    S0, S = cfg.max_prefill, cfg.max_chunk
    cache.prefill(rnd(B, Hq, S0, d), rnd(B, Hkv, S0, d), rnd(B, Hkv, S0, d))
    for _ in range(n_steps):
        cache.chunk_step(rnd(B, Hq, S, d), rnd(B, Hkv, S, d), rnd(B, Hkv, S, d))
    torch.cuda.synchronize()
    return cache


def test_normal_steps_never_reach_the_bound(monkeypatch):
    monkeypatch.delenv("H2O_SELECT_SPIN_LIMIT", raising=False)
    monkeypatch.delenv("H2O_SELECT_SYNC_SKEW", raising=False)
    h2o = h2o_mod()
    # 384-token chunks: 12 parts per head; evicting from the second step on
    cfg = h2o.H2OConfig(2, 8, 2, 64, 640, 32, 384, 512, "bf16")
    cache = _steps(h2o, cfg, 6, seed=1)
    assert h2o.h2o_device_status(cache.handle) == 0
    assert int(cache.positions.max()) >= cfg.cache_slots
    cache.close()


def test_unsatisfiable_wait_ends_and_sets_the_flag(monkeypatch):
    monkeypatch.setenv("H2O_SELECT_SPIN_LIMIT", "4")
    monkeypatch.setenv("H2O_SELECT_SYNC_SKEW", "1")
    h2o = h2o_mod()
    cfg = h2o.H2OConfig(1, 4, 2, 64, 640, 32, 384, 512, "bf16")
    cache = _steps(h2o, cfg, 2, seed=2)
    assert h2o.h2o_device_status(cache.handle) == 2
    assert h2o.h2o_device_status(cache.handle) == 0         # cleared by the read
    cache.close()
    # the knobs are read when a handle is made: a new one without them waits normally
    monkeypatch.delenv("H2O_SELECT_SPIN_LIMIT")
    monkeypatch.delenv("H2O_SELECT_SYNC_SKEW")
    cache = _steps(h2o, cfg, 2, seed=2)
    assert h2o.h2o_device_status(cache.handle) == 0
    cache.close()
