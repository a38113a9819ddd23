"""MI355X (gfx950) routed MoE expert-FFN layer: stable route alignment,
packed int4 AWQ-style gate/up with SiLU(gate)*up, down projection and the
router-weighted top-k combine, as hand-written HIP kernels behind a C ABI
(include/moe_ffn.h). This package is the thin Python binding over it.
"""
from ._binding import (  # noqa: F401
    MOE_ERR_CAPACITY,
    MOE_ERR_HIP,
    MOE_ERR_INVALID_ARG,
    MOE_ERR_UNSUPPORTED,
    MOE_ERR_WORKSPACE,
    MOE_OK,
    MOE_PATH_AUTO,
    MOE_PATH_DECODE,
    MOE_PATH_GROUPED,
    MOE_W_INT4_AWQ,
    MOE_W_MXFP8,
    MoeError,
    declared_symbols,
    lib,
    make_desc,
    moe_align,
    moe_align_capacity,
    moe_ffn_auto_decode_max_m,
    moe_ffn_desc,
    moe_ffn_down_combine,
    moe_ffn_forward,
    moe_ffn_forward_aligned,
    moe_ffn_forward_profiled,
    moe_ffn_gate_up,
    moe_ffn_intermediate,
    moe_ffn_kernel_count,
    moe_ffn_kernel_name,
    moe_ffn_workspace_size,
    moe_weights,
    status_str,
    weights_struct,
)
from .layer import DeviceProjection, MoeLayer  # noqa: F401
