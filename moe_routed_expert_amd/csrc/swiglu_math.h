// Element math of the clamped SwiGLU forward, shared by the streaming kernels
// and the grouped-GEMM epilogue so that both compute the same bits.
//
// Operation (page "nemo_automodel.components.moe.swiglu_triton", module
// description): y = silu(min(gate, L)) * clamp(up, -L, L) * p in fp32, the
// product taken left to right. Clamps are compare/select, so NaN passes
// through as in torch.clamp; exp is v_exp_f32 of -z * log2(e) and 1/(1+e) is
// v_rcp_f32; the rest are fp32 multiplies (the library is built with
// -ffp-contract=off, so none is fused).
#pragma once

#include <hip/hip_runtime.h>

namespace moe_epi {

// sigma(z) = 1 / (1 + e^-z) with e^-z = 2^(-z * log2(e)).
// v_rcp_f32 returns no subnormal results: for z in about (-88.7, -87.3] the
// true 1/(1 + e) lies below 2^-126 and would come back as 0, turning silu(z)
// (a normal number there, z times that subnormal) into a zero. So the
// reciprocal is taken of (1 + e) * 2^-32, which keeps it normal for every
// finite 1 + e, and scaled back by 2^-32: both scalings are exact above
// 2^-126, and below it the final multiply rounds into the subnormal range as
// IEEE division would (the kernels run with fp32 subnormals enabled).
__device__ __forceinline__ float sigmoid_f32(float z) {
    const float e = __builtin_amdgcn_exp2f(z * -1.4426950408889634f);
    return __builtin_amdgcn_rcpf((1.0f + e) * 0x1p-32f) * 0x1p-32f;
}

// clamp(gate, max=L): a comparison with NaN is false, so NaN passes through.
__device__ __forceinline__ float clamp_hi(float g, float L) { return (g > L) ? L : g; }

// clamp(up, -L, L), NaN passes through.
__device__ __forceinline__ float clamp_sym(float u, float L) {
    return (fabsf(u) > L) ? copysignf(L, u) : u;
}

__device__ __forceinline__ float fwd_elem(float g, float u, float p, float L) {
    const float gc = clamp_hi(g, L);
    const float uc = clamp_sym(u, L);
    const float s = sigmoid_f32(gc);
    return ((gc * s) * uc) * p;
}

}  // namespace moe_epi
