"""Split-KV PagedAttention decode for AMD MI355X (gfx950).

The compute lives in ``libpagedattn.so`` (hand-written HIP kernels behind a
C ABI, declared in ``include/pagedattn.h``).
"""
