"""Split-KV PagedAttention decode for AMD MI355X (gfx950).

The compute lives in ``libpagedattn.so`` (hand-written HIP kernels behind a
C ABI, declared in ``include/pagedattn.h``). The functions exported here only
marshal torch tensors into that ABI; importing the package does not load the
library, the first call does (and raises if it is missing).
"""
from .api import (  # noqa: F401
    PagedAttnError,
    build_page_indices,
    library_path,
    load_library,
    normal_decode_set_metadata,
    num_kv_splits,
    paged_attn_decode,
    paged_attn_decode_kernel,
    paged_attn_decode_static,
    paged_attn_reduce,
    paged_token_offsets,
    prepare_swa_spec_page_table,
)
