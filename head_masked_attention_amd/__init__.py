"""libbsattn: content-aware block-sparse, head-masked self-attention on MI355X.

Python binding over the C ABI declared in include/bsattn.h.  The kernels are
hand-written HIP for gfx950; this package only marshals torch tensors (device
memory and streams) into the C calls.
"""
from ._binding import (  # noqa: F401
    BF16,
    DECLINE_CAUSAL,
    DECLINE_DISABLED,
    DECLINE_EXCLUDED,
    DECLINE_NO_BACKEND,
    DECLINE_NOT_SELF,
    DECLINE_SHORT,
    DECLINE_TOKEN_MASK,
    DEFAULT_MIN_LENGTH,
    DEFAULT_SPARSITY,
    EXPORTS,
    F32,
    LIB_PATH,
    MAX_SEGMENTS,
    MIN_ACTIVE_HEADS,
    NOTE_NO_LAYOUT,
    NOTE_NONE,
    SEG_KINDS,
    STAGE_SPARSE,
    Stage,
    BlockMask,
    BsattnError,
    Layout,
    budget_k,
    empty_block_mask,
    forward,
    head_mask,
    layout_classes,
    load_library,
    mask_density,
    radial,
    select,
    select_workspace_bytes,
    status_string,
)
