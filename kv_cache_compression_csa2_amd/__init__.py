"""CSA2 (Compressed Sparse Attention 2) global-attention hot path for MI355X.

HIP kernels for gfx950 behind a C ABI (include/csa2.h, built into libcsa2.so);
this package binds it with ctypes (argument marshalling only) and supplies the
seeded synthetic workloads and the per-step call sequence.
"""
from ._lib import (Csa2Error, csa2_index_full, csa2_index_prefill_topk,  # noqa: F401
                   csa2_index_prefill_topk_workspace_bytes, csa2_index_reindex, csa2_index_reindex_topk,
                   csa2_index_reindex_topk_workspace_bytes, csa2_index_topk, csa2_index_topk_noalloc,
                   csa2_index_topk_merge_pool, csa2_index_topk_noalloc_scratch_bytes,
                   csa2_index_topk_pool_workspace_bytes, csa2_index_topk_workspace_bytes, csa2_sparse_attn,
                   csa2_sparse_attn_workspace_bytes, csa2_topk, csa2_topk_workspace_bytes, format_version,
                   fp4_kv_pack, fp4_kv_unpack, kidx_fp4_pack, load, swa_fp8_pack)
