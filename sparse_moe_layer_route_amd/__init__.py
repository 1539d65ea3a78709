"""MI355X (gfx950) MoE layer forward: HIP kernels behind a C ABI
(include/moe_route.h), with a thin ctypes binding of the same names."""
from .binding import (  # noqa: F401
    Dims, MoEError, MoeDims, MoeWeights, MoeDebug, MODES, EXPORTED, LIB_PATH,
    moe_abi_version, moe_workspace_size, moe_route, moe_prefetch_mask, moe_prefetch_adaptive,
    moe_pack_size, moe_pack_weights, pack_weights, LAYOUTS, moe_permute,
    moe_floe_predict, moe_floe_pack, moe_lore_targets, moe_lore_fit_size, moe_lore_fit,
    moe_expert_ffn, moe_lore_surrogate, moe_combine, moe_layer_forward, weights_struct,
    moe_layer_forward_noalloc, NOALLOC_SCRATCH_BYTES,
    MoeOffloadCost, MoeOffloadStats, OFFLOAD_NONE, OFFLOAD_FETCH, OFFLOAD_HOST, offload_cost,
    moe_offload_plan, moe_offload_workspace_size, moe_host_ffn_workspace_size,
    moe_host_expert_ffn, moe_layer_forward_offload,
)
