"""LongCat Sparse Attention (LSA) hot path on MI355X (gfx950).

The compute lives in liblsa.so (hand-written HIP kernels behind the C ABI in
include/lsa.h); this package is its thin Python binding plus the workload
definitions and the seeded synthetic input generator.
"""
from ._lib import (  # noqa: F401
    LSAError,
    LSAUnavailable,
    lsa_block_summary,
    lsa_hier_select,
    lsa_index_score,
    lsa_select_topk,
    lsa_sparse_attn_decode,
    lsa_sparse_attn_prefill,
    load,
    status_string,
)
