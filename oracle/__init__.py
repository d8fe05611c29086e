"""CPU oracle for paged, quantized-KV decode/verify attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, table
or constant generator with the HIP library under
``paged_quantized_kv_ra_amd/``.

Everything here is plain numpy, in float64 wherever the method leaves the
precision open, written to be read against the pages it follows:

* ``codecs``    -- the KV element formats (FP16, FP8 E4M3, INT8) with
                   per-layer scalar scales, and their exact dequantisation.
* ``layout``    -- the paged cache's byte layout (the library's documented
                   ABI), scatter of new tokens into pages and gather back.
* ``attention`` -- softmax attention of a query block over dequantised,
                   contiguous (unpaged) KV, the split-KV partials and the
                   log-sum-exp merge.

Parity status of each function is stated in its module header.
"""
