"""MI355X-native channels-last GroupNorm with optional fused SiLU.

The compute lives in libgnsilu.so (hand-written HIP for gfx950, C ABI in
include/gnsilu.h); this package is its Python binding.
"""
from .binding import (  # noqa: F401
    GnDtype,
    GnStatus,
    LIB_PATH,
    MAX_CHANNELS,
    apply_rows,
    conv3x3,
    conv_plan,
    dtype_code,
    gn_apply_rows,
    gn_apply_rows_dtype,
    gn_conv3x3_nhwc,
    gn_conv3x3_plan,
    gn_kernel_name,
    gn_plan_rows,
    gn_plan_rows_dtype,
    gn_profile_rows,
    gn_profile_rows_dtype,
    gn_silu_ndhwc,
    gn_silu_ndhwc_dtype,
    gn_silu_ndhwc_strided_dtype,
    gn_silu_nhwc,
    gn_silu_nhwc_dtype,
    gn_silu_nhwc_strided,
    gn_silu_nhwc_strided_dtype,
    gn_silu_rows,
    gn_silu_rows_dtype,
    gn_stats_rows,
    gn_stats_rows_dtype,
    gn_status_string,
    gn_version,
    group_norm_silu_4d,
    group_norm_silu_5d,
    group_norm_silu_rows,
    group_stats_rows,
    lib,
    plan_rows,
    profile_rows,
    status_text,
)

__version__ = "0.1.0"
