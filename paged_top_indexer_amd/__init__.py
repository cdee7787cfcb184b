"""MI355X-native QSA sparse-attention decode: paged top-512 block selection
and sparse attention over the selected tokens, as hand-written HIP kernels
for gfx950 behind a small C ABI (``include/qsa.h``).

The entry points carry the C names; the library is loaded on first
use and there is no fallback path.
"""

from ._binding import (  # noqa: F401
    COMPRESS_RATIO,
    OUT_WIDTH,
    TOKEN_TOPK,
    TOPK_BLOCKS,
    constants,
    decode_step_workspace_bytes,
    kv_views,
    library,
    build_metadata_workspace_bytes,
    qsa_build_metadata,
    qsa_decode_step,
    qsa_decode_step_fp8,
    qsa_decode_step_noalloc,
    qsa_paged_logits,
    qsa_select,
    qsa_select_fp8,
    qsa_select_weighted,
    qsa_topk_per_row,
    qsa_sparse_attn,
    select_workspace_bytes,
    sparse_attn_workspace_bytes,
    topk_per_row_workspace_bytes,
)
