"""MI355X-native HelixLinear (HXQ) forward pass.

The compute lives in libhxq (HIP kernels for gfx950 behind the C ABI declared
in include/hxq.h); this package is its Python binding plus a thin layer
object.  Importing it does not load the library; the first call does, and
raises if the library has not been built.
"""

from ._binding import (  # noqa: F401
    HXQ_BF16,
    HXQ_F32,
    HXQ_FMT_PK12,
    HXQ_FMT_U8,
    HXQ_MAX_GROUP,
    HXQ_VARIANT_AUTO,
    HXQ_VARIANT_GEMM_BF16,
    HXQ_VARIANT_GEMM_BF16_T256,
    HXQ_VARIANT_GEMV_MFMA,
    HXQ_VARIANT_GEMV_VALU,
    HXQ_VARIANT_GENERIC,
    VARIANT_NAMES,
    HxqBwdLayer,
    HxqError,
    HxqLayer,
    hxq_dequant_bf16,
    hxq_linear_bwd_x,
    hxq_linear_bwd_x_grouped,
    hxq_linear_bwd_x_noalloc,
    hxq_linear_bwd_x_workspace,
    hxq_linear_fwd_grouped,
    hxq_linear_fwd_pk12,
    hxq_linear_fwd_u8,
    hxq_linear_fwd_ws,
    hxq_select_variant,
    hxq_sidecar_add,
    hxq_version,
    lib,
)
from .layer import HelixLinear  # noqa: F401
