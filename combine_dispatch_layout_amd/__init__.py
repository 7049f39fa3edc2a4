"""MI355X (gfx950) hot path of MoE token dispatch and combine for one
expert-parallel rank: routing layout, normal / low-latency / fp8 row scatter
and the top-k-weighted gather-combine, as HIP kernels behind the C ABI in
``include/cdl.h``.  ``api`` is the thin Python binding; ``workloads`` draws
seeded synthetic inputs.
"""
from .api import (  # noqa: F401
    CDL_ERR_SCRATCH,
    NOALLOC_SCRATCH_BYTES,
    CDL_STATUS_LL_OVERFLOW,
    CDL_STATUS_MAP_RANGE,
    CDL_STATUS_REORDER_OVERFLOW,
    CDL_STATUS_ROWS_OVERFLOW,
    FP8_GROUP,
    FP8_SCALE_COLMAJOR,
    FP8_SCALE_PACKED,
    FP8_SCALE_UE8M0,
    LIB_PATH,
    CdlError,
    Layout,
    combine,
    dispatch,
    dispatch_fp8,
    dispatch_layout,
    dispatch_ll,
    dispatch_ll_fp8,
    fp8_scale_bytes,
    new_scale_tensor,
    layout_workspace_size,
    library,
    ll_expected_m,
    permute,
    permute_ll,
    permute_ll_fp8,
    permute_fp8,
    permute_fp8_tensor,
    permute_fp8_workspace_size,
    rank_layout,
    RankLayout,
    status_string,
)
