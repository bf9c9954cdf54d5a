"""CPU oracle for paged KV-cache decode: test infrastructure, not product code.

Only the tests, the smoke check in ``__graft_entry__`` and the CPU-baseline leg
of ``bench.py`` may import anything from here.  The HIP library never calls
into this package and this package never calls into the HIP library; the only
code both sides share is the seeded input generator package ``workloads``.

Modules (each function cites the passage of the source pages it follows):

* ``layout``          - the oracle's own reader/writer of the physical cache
                        layout (defined in ``include/pagedkv.h``).
* ``attention``       - decode attention written as its plain definition: gather
                        a sequence's blocks into contiguous K/V, then textbook
                        softmax attention in float64.
* ``cache``           - the cache write (scatter of new tokens into their slots)
                        and the whole-block copy used for copy-on-write.
* ``allocator_model`` - the block manager: FIFO free list, per-sequence block
                        tables, reference counts, fork and copy-on-write.
* ``scheduler_model`` - the continuous-batching loop that drives the allocator
                        over a serving trace.

Pins (what ties each part to something other than itself) are listed in the
module headers; every module here is pinned by the ``-m "not gpu"`` tests.
"""
