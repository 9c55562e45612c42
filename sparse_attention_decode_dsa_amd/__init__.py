"""MI355X-native DSA sparse decode step: fp8 indexer, exact top-k with a
per-split local selection and exact merge, split-K sparse absorbed-MLA
attention over paged fp8 rows, and the natural-log LSE merge.

The kernels are hand-written HIP for gfx950 in ``csrc/`` behind the C ABI of
``include/dsa.h`` (``libdsa.so``).  ``sparse_attention_decode_dsa_amd.dsa``
is the thin Python binding with the same names; ``workload`` makes seeded
synthetic inputs.  Importing this package loads nothing native.
"""

__all__ = ["dsa", "workload"]
