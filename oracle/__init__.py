"""CPU oracle of the chunked H2O attention step (fp64 numpy + a pure-Python brute force).

TEST INFRASTRUCTURE ONLY: importable by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product package
``kv_cache_eviction_amd``, with which it shares no code.
"""
