"""MI355X-native routed-expert epilogue: clamped SwiGLU x routing probability and the
fp32 router-weight multiply, each with a forward and a single-pass backward, and the
gate_up grouped GEMM with the clamped SwiGLU epilogue fused into it (bf16 MFMA),
the down-projection grouped GEMM with the router-weight multiply fused into it,
and the fp32 combine of routed rows into tokens, as hand-written HIP kernels for
gfx950 behind a C ABI (include/moe_epi.h).

The binding loads libmoe_epi.so on first use and raises if it is not built.
"""
from .binding import (MoeEpiError, RouterWeightMul, SwigluClamped, grouped_down_router_fwd,
                      grouped_gate_up_swiglu_fwd, moe_combine_fwd, router_weight_mul,
                      router_weight_mul_bwd, router_weight_mul_fwd, swiglu_clamped,
                      swiglu_clamped_bwd, swiglu_clamped_fwd)

__all__ = [
    "MoeEpiError", "RouterWeightMul", "SwigluClamped", "grouped_down_router_fwd", "grouped_gate_up_swiglu_fwd",
    "moe_combine_fwd", "router_weight_mul",
    "router_weight_mul_bwd",
    "router_weight_mul_fwd", "swiglu_clamped", "swiglu_clamped_bwd", "swiglu_clamped_fwd",
]
