"""Oracle for paged decode attention — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct CPU statement of what the hot path computes:

* ``attention``      fp64 single-query softmax attention over each sequence's
                     contiguous K/V (no blocks, no tables);
* ``allocator_model`` the block allocator's policy (free pool, reference
                     counts, copy-on-write, release at zero) as a pure-Python
                     model;
* ``paged_layout``   where a token's K/V elements live inside the paged cache,
                     and what ``kv_append`` / ``block_copy`` must leave there.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``paged_kv_cache_358_amd``) and imports nothing from it; its only shared
dependency is the seeded input module ``synth``.

Parity pins (tests/test_oracle_*.py, run with ``-m "not gpu"``) tie each
function to facts the pages and the mathematics fix.  No function here is
"parity unpinned".
"""
