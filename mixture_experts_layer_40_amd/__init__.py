"""libmoe: the DeepSeekMoE layer forward pass on AMD Instinct MI355X (gfx950).

The compute lives in libmoe.so (hand-written HIP kernels behind the C ABI of
include/libmoe.h); this package is its thin Python binding with the same
function names, plus MoELayer, which holds a layer's buffers and enqueues
the call sequence. Build the library with
`python -m mixture_experts_layer_40_amd.build`.
"""

from ._lib import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    MOE_DTYPE_BF16,
    MOE_DTYPE_F32,
    MOE_DTYPE_FP8_E4M3,
    MOE_ERR_DTYPE,
    MOE_ERR_HIP,
    MOE_ERR_NULL,
    MOE_ERR_SHAPE,
    MOE_ERR_UNSUPPORTED,
    MOE_ERR_WORKSPACE,
    MOE_LAYOUT_ROWS,
    MOE_LAYOUT_TILED,
    MOE_NORM_NONE,
    MOE_NORM_ONE_PLUS_SELECTED,
    MOE_NORM_SELECTED,
    MOE_OK,
    MOE_PACK_DOWN,
    MOE_PACK_GATE_UP,
    MOE_SCORE_SIGMOID,
    MOE_SCORE_SOFTMAX,
    MOE_WS_EXPERTS,
    MOE_WS_FFN,
    MOE_WS_GEMM,
    MOE_WS_PERMUTE,
    MOE_WS_ROUTE,
    MOE_WS_SHARED,
    MoEError,
    config_of,
    load_library,
    make_config,
    moe_bias_update,
    moe_combine,
    moe_combine_residual,
    moe_config,
    moe_expert_down,
    moe_expert_ffn,
    moe_expert_gate_up,
    moe_experts,
    moe_experts_down,
    moe_experts_gate_up,
    moe_pack_weights,
    moe_permute,
    moe_rmsnorm,
    moe_route,
    moe_sequence_loads,
    moe_shared_ffn,
    moe_status_string,
    moe_validate,
    moe_workspace_size,
    pack_down,
    pack_gate_up,
)
from .layer import MoELayer  # noqa: F401
