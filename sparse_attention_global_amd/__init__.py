"""MI355X-native global cross-frame attention layer (dense, Speed3R GSA, AVGGT
subsampled) -- Python binding of the HIP library libsga.so."""
from ._lib import (  # noqa: F401
    EXPORTS, SGA_BF16, SGA_F32, compact_rows, dense_global_attn, dense_workspace_bytes,
    SGA_KEEP_REF_FRAME, SGA_KEEP_SPECIAL, fine_workspace_bytes, gsa_compress,
    gsa_compressed_pooled, gsa_gate, pooled_workspace_bytes,
    gsa_layer, gsa_select_topk, gsa_select_topk_noalloc, gsa_select_topk_probability, gsa_sparse_attn, gsa_sparse_attn_gated, keep_flags, library, pooled_shape, sga_compact,
    subsampled_global_attn, tokens, topk_prob_workspace_bytes, topk_workspace_bytes, workspace_bytes,
)

__version__ = "0.1.0"
