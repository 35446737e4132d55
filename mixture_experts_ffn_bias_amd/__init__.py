"""DeepSeek-V3.2-Exp MoE layer forward for one AMD MI355X (gfx950).

The layer runs in hand-written HIP kernels behind the C ABI of include/moe.h
(libmoe.so, built by ``python -m mixture_experts_ffn_bias_amd.build``); this
package is its Python binding.
"""
from ._binding import (  # noqa: F401
    FUSED_MAX_TOKENS, LIB_PATH, MOE_ERR_STALLED, MOE_FORWARD_EVENTS, MOE_STATIC_WORKSPACE_BYTES, SYMBOLS, MoeError,
    MoELayer, experts_struct, experts_struct_bf16, fused_workspace, lib, make_dims, mlp_workspace, moe_add_rmsnorm,
    moe_combine, moe_dims, moe_experts, moe_experts_bf16, moe_forward, moe_forward_bf16, moe_forward_bf16_timed,
    moe_forward_fused, moe_forward_fused_status, moe_forward_fused_workspace_size, moe_forward_no_workspace,
    moe_forward_shard, moe_forward_timed, moe_gate, moe_grouped_ffn, moe_grouped_ffn_bf16, moe_mlp,
    moe_mlp_workspace_size, moe_permute, moe_weights, moe_weights_bf16, moe_workspace_size, status_string, workspace,
)
