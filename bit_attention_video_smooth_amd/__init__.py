"""bit_attention_video_smooth_amd: FP8 (E4M3) smoothed attention for AMD MI355X.

The compute path is libvsmooth.so (HIP kernels for gfx950, C ABI in
include/vsmooth.h); this package only marshals PyTorch tensors to it.  The
library is loaded on first use and a missing build raises.
"""
from .api import (Plan, attention, vs_cube_permutation, vs_fp8_attn_fwd,  # noqa: F401
                  vs_fp8_attn_fwd_pcodes,
                  vs_kmeans_permute,
                  vs_kmeans_workspace_bytes, vs_quantize_residual, vs_quantize_residual_ex,
                  vs_quantize_residual_perm,
                  vs_smooth_stats, vs_smooth_stats_ex, vs_smooth_stats_noalloc,
                  vs_smooth_stats_workspace_bytes, vs_version)
from ._abi import (VS_EXPCAST, VS_OUT_BF16, VS_BF16_MMA, VS_QK_HADAMARD, VS_V_MXFP4, VS_LAYOUT_BHSD, VS_LAYOUT_BSHD, VS_VMEAN_BLOCK,  # noqa: F401
                   VS_VMEAN_BLOCK_OUT, VS_VMEAN_NONE, VS_VMEAN_SEQ, VsError, LIB_PATH)
