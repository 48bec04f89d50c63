"""Block-draft verify pass for MI355X (gfx950).

The compute lives in libspecverify.so (hand-written HIP, C ABI in
include/spec_verify.h); this package is its thin Python binding.
"""
from ._binding import (  # noqa: F401
    BLOCK, DERR_CAPACITY, DERR_COMMIT, DERR_LENGTH, DERR_PAGE, DERR_RANGE, DERR_TOKEN, EXPORTS, KERNEL_KINDS, LIB_PATH,
    WFMT_BF16, WFMT_FP8_E4M3_ROW, WFMT_MXFP4, ACT_FMTS, DeviceModel, SpecError, Verifier, debug_attention,
    debug_linear, debug_linear_mx8, debug_quant_mx8, debug_residual, debug_rmsnorm, debug_swiglu, load_library)
