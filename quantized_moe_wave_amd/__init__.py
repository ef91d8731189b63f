"""Routed-expert MoE FFN layer (Q4_K experts) for MI355X / gfx950.

The layer runs in hand-written HIP kernels behind the C ABI of
include/moe_ffn.h; this package is a thin ctypes binding with the same names.
"""
from .binding import (  # noqa: F401
    MoeError,
    STAT_FIELDS,
    STAT_STAGES,
    MoeFfn,
    abi_version,
    moe_ffn_create,
    moe_ffn_debug_routing,
    moe_ffn_debug_stats,
    moe_ffn_destroy,
    moe_ffn_forward,
    moe_ffn_forward_block,
    moe_ffn_forward_noalloc,
    moe_ffn_forward_q8,
    moe_ffn_profile,
    moe_ffn_profile_read,
    moe_ffn_stage_names,
    moe_ffn_reserve,
    moe_ffn_set_norm,
)
