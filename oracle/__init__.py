"""CPU oracle for the paged decode path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
in ``paged_kv_cache_381_amd`` and never imports it.
"""
