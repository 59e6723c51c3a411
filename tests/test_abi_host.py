"""Host-only checks of the C ABI library: it loads, exports every symbol that
include/h2o.h declares, and validates configs (no GPU call is made)."""
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib_module():
    from kv_cache_eviction_amd import build_lib
    if not os.path.exists(build_lib.LIB):
        build_lib.build(verbose=False)
    from kv_cache_eviction_amd import h2o
    return h2o


def _declared():
    text = open(os.path.join(ROOT, "include", "h2o.h")).read()
    return sorted(set(re.findall(r"H2O_API\s+[\w\s\*]+?\b(h2o_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    h2o = _lib_module()
    declared = _declared()
    assert len(declared) >= 15
    assert sorted(h2o.EXPORTED) == declared
    for name in declared:
        assert hasattr(h2o._lib, name), name


def _cfg(**kw):
    h2o = _lib_module()
    base = dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, cache_slots=2048,
                recent_window=256, max_chunk=1024, max_prefill=2048, dtype="bf16")
    base.update(kw)
    return h2o.H2OConfig(**base)


def test_named_workload_configs_validate():
    h2o = _lib_module()
    from kv_cache_eviction_amd.workloads import WORKLOADS
    for w in WORKLOADS.values():
        cfg = h2o.H2OConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.cache_slots,
                            w.recent_window, w.chunk, w.prefill, w.dtype)
        assert h2o.h2o_validate_config(cfg) == h2o.H2O_OK, w.name
        assert h2o.h2o_workspace_bytes(cfg) > 0


@pytest.mark.parametrize("kw", [
    dict(n_q_heads=30),                 # Hq % Hkv != 0
    dict(head_dim=96),
    dict(dtype_code=9),
    dict(recent_window=1500),           # M - W < max_chunk
    dict(max_prefill=4096),             # > M
    dict(cache_slots=20000),
    dict(batch=0),
    dict(max_chunk=0),
    dict(recent_window=-1),
    dict(softmax_scale=math.nan),
    dict(n_q_heads=1024, n_kv_heads=1),  # G * max_len above 2^20 query rows per KV group
    dict(policy="bogus"),
    dict(n_sink=4),                     # sinks only with the sink_recent policy
    dict(policy="sink_recent", n_sink=-1),
    dict(policy="sink_recent", n_sink=900),   # M - W - n_sink < max_chunk
])
def test_invalid_configs_are_rejected(kw):
    h2o = _lib_module()
    if "dtype_code" in kw:
        c = _cfg().c()
        c.dtype = kw["dtype_code"]
        import ctypes
        assert h2o._lib.h2o_validate_config(ctypes.byref(c)) == h2o.H2O_ERR_CONFIG
        assert h2o._lib.h2o_workspace_bytes(ctypes.byref(c)) == 0
        return
    cfg = _cfg(**kw)
    assert h2o.h2o_validate_config(cfg) == h2o.H2O_ERR_CONFIG
    assert h2o.h2o_workspace_bytes(cfg) == 0


def test_null_config_and_status_strings():
    h2o = _lib_module()
    assert h2o._lib.h2o_validate_config(None) == h2o.H2O_ERR_NULL
    for s in range(9):
        assert h2o.status_str(s) and h2o.status_str(s) != "unknown status"
    assert h2o.status_str(99) == "unknown status"


def test_null_handle_calls_fail_cleanly():
    h2o = _lib_module()
    assert h2o._lib.h2o_prefill(None, None, None, None, 4, None, None, None) == h2o.H2O_ERR_NULL
    assert h2o._lib.h2o_chunk_step(None, None, None, None, 4, None, None, None, None, None, None,
                                   None, None) == h2o.H2O_ERR_NULL
    assert h2o._lib.h2o_recurrence_backward_step(*([None] * 11), 4, *([None] * 9), 0, None) == h2o.H2O_ERR_NULL
    assert h2o._lib.h2o_tokens_seen(None) == -1
    assert h2o._lib.h2o_last_hip_error(None) == 0


def test_misaligned_buffer_pointers_are_refused():
    """A buffer pointer off a 16-byte boundary is refused on the host before
    anything is enqueued (the fake addresses below are never dereferenced)."""
    import ctypes
    h2o = _lib_module()
    c = _cfg().c()
    good, bad = 0x10000, 0x10008
    ws = h2o._lib.h2o_workspace_bytes(ctypes.byref(c))
    for i in range(5):      # k_cache, v_cache, scores, positions, workspace
        p = [good] * 5
        p[i] = bad
        out = ctypes.c_void_p(0x20000)
        assert h2o._lib.h2o_cache_init(ctypes.byref(c), *p, ws, 0, 0, None,
                                       ctypes.byref(out)) == h2o.H2O_ERR_ALIGN
        assert out.value is None
    for i in range(15):     # q .. v_new, then out .. workspace
        p = [good] * 15
        p[i] = bad
        assert h2o._lib.h2o_chunk_backward(ctypes.byref(c), *p[:6], 64, *p[6:], 1 << 40,
                                           None) == h2o.H2O_ERR_ALIGN
    for i in range(19):     # k_cache .. v_new, then out .. workspace
        p = [good] * 19
        p[i] = bad
        assert h2o._lib.h2o_recurrence_backward_step(ctypes.byref(c), *p[:10], 64, *p[10:], 1 << 40,
                                                     None) == h2o.H2O_ERR_ALIGN
    assert "aligned" in h2o.status_str(h2o.H2O_ERR_ALIGN)


def test_position_policy_configs_validate():
    h2o = _lib_module()
    assert h2o.h2o_validate_config(_cfg(policy="recent")) == h2o.H2O_OK
    assert h2o.h2o_validate_config(_cfg(policy="sink_recent", n_sink=4)) == h2o.H2O_OK
    assert h2o.h2o_validate_config(_cfg(policy="sink_recent", n_sink=768)) == h2o.H2O_OK
