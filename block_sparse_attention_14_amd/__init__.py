"""Sol-Attn sparse attention forward for AMD Instinct MI355X (gfx950).

The work is done by libsolattn.so (HIP kernels behind the C ABI in
include/sol_attn.h); this package only loads it and marshals torch tensors.
Importing the package does not load the library; the first call does, and it
raises if the library has not been built.
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    SOL_ATTN_MAX_N,
    SOL_ATTN_SCRATCH_BYTES,
    SOL_EHIP,
    SOL_EINVAL,
    SOL_ESCRATCH,
    SOL_EUNSUPPORTED,
    SOL_EWORKSPACE,
    SOL_F_EXACT_ONLY,
    SOL_F_GROUP2,
    SOL_F_GROUP4,
    SOL_F_GROUP8,
    SOL_F_GROUP16,
    SOL_F_GROUP6,
    SOL_F_OUT_BF16,
    SOL_F_PLANNED,
    SOL_F_POOLED,
    SOL_F_PREPARED,
    SOL_F_ROW_CORRECTION,
    SOL_OK,
    SOL_ROUTE_GAUSS,
    SOL_ROUTE_GAUSS_DIAG,
    SOL_ROUTE_ROWMAX,
    SolAttnError,
    lib,
    strerror,
)
from .api import (  # noqa: F401
    MaskBuilder,
    SolAttention,
    bitmap_shape,
    forward,
    forward_noalloc,
    new_stats,
    pool,
    pooled_shape,
    read_stats,
    unpack_bitmap,
    workspace_bytes,
)
