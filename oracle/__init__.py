"""CPU oracle for ragged-paged decode attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct reference implementations written from the
pages, never from the HIP library:

* ``planner``   -- integer admission work: per-head budget reservation,
                   clustering, tier split, the ref-counted page allocator,
                   block tables and the split plan (all exact integers).
* ``quant``     -- the slow tier's block-wise symmetric INT8 quantiser.
* ``attention`` -- fp64 decode attention over each head's retained rows, and
                   the log-sum-exp merge of partial results.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything here.  The product path
(``non_uniform_paged_amd``) never does, and this package imports nothing from
it; the two share only the seeded input generators in ``workloads``.

Pinning status of each function is stated in its module header.
"""
