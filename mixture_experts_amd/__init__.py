"""MI355X-native DeepSeek-V3-style MoE layer forward: C-ABI library of gfx950 HIP
kernels (libmoe_mi355x.so, include/moe.h) and its thin Python binding."""
from ._lib import (EXPORTS, FLAT_LIB_PATH, KERNEL_TAGS, LIB_PATH, MoeConfig, MoeError, MoeWeights, RECIPE_BF16, RECIPE_F32,
                   RECIPE_FP8_B128, RECIPE_MXFP4, RECIPE_NVFP4, SCORE_SIGMOID, SCORE_SQRTSOFTPLUS, library, load, make_config,
                   make_expert_weights, make_weights, moe_combine, moe_convert_mxfp4_to_fp8, moe_forward, moe_forward_noalloc,
                   moe_forward_noalloc_scratch_bytes, moe_forward_residual, moe_grouped_ffn,
                   moe_pack_fp4_scales, moe_permute, moe_profile_start, moe_profile_stop, moe_rmsnorm, moe_route,
                   moe_workspace_bytes, pack_fp4_scales)
from .layer import MoELayerBuffers, alloc_buffers
