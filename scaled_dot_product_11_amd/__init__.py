"""MI355X-native fused scaled-dot-product attention: forward and gradients.

The computation runs in hand-written HIP kernels for gfx950 behind the C ABI declared in
include/sdpa.h; this package is its thin Python binding (names mirror the C entry points).
"""
from ._binding import (EXPORTS, LIB_PATH, SDPA_BF16, SDPA_CAUSAL_BOTTOM_RIGHT, SDPA_CAUSAL_NONE,
                       SDPA_CAUSAL_TOP_LEFT, SDPA_F16, SDPA_F32, SDPA_STATIC_WORKSPACE_BYTES,
                       STATUS_NAMES, SdpaError, SdpaPlan,
                       load_library, sdpa_bwd, sdpa_bwd_bias, sdpa_bwd_bias_check,
                       sdpa_bwd_check, sdpa_bwd_varlen, sdpa_bwd_varlen_check, sdpa_check, sdpa_fwd,
                       sdpa_fwd_bias, sdpa_fwd_bias_check, sdpa_fwd_splitkv,
                       sdpa_fwd_splitkv_check, sdpa_fwd_splitkv_noalloc,
                       sdpa_fwd_splitkv_workspace, sdpa_fwd_varlen,
                       sdpa_fwd_varlen_check, sdpa_plan, sdpa_plan_item, sdpa_strerror)

__all__ = ["sdpa_fwd", "sdpa_check", "sdpa_fwd_bias", "sdpa_fwd_bias_check", "sdpa_fwd_splitkv",
           "sdpa_fwd_splitkv_check", "sdpa_fwd_splitkv_noalloc", "sdpa_fwd_splitkv_workspace",
           "sdpa_fwd_varlen",
           "sdpa_fwd_varlen_check", "sdpa_bwd", "sdpa_bwd_check", "sdpa_bwd_bias",
           "sdpa_bwd_bias_check", "sdpa_bwd_varlen", "sdpa_bwd_varlen_check", "sdpa_strerror", "sdpa_plan",
           "sdpa_plan_item", "SdpaError", "SdpaPlan", "SDPA_F32", "SDPA_BF16", "SDPA_F16",
           "SDPA_CAUSAL_NONE", "SDPA_CAUSAL_TOP_LEFT", "SDPA_CAUSAL_BOTTOM_RIGHT", "STATUS_NAMES",
           "SDPA_STATIC_WORKSPACE_BYTES",
           "LIB_PATH", "EXPORTS", "load_library"]
