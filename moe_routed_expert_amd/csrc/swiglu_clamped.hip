// Clamped SwiGLU times routing probability: forward and single-pass backward
// for gfx950.
//
// Operation (page "nemo_automodel.components.moe.swiglu_triton", module
// description): on the grouped-GEMM output x = [gate | up] (bf16,
// [rows, 2*inter]) with one fp32 probability per row,
//   y = silu(min(gate, L)) * clamp(up, -L, L) * p,
// computed in fp32 and rounded once to bf16. The backward writes d_gate and
// d_up into the two halves of grad_x and reduces the per-row probability
// gradient in registers; its clamp gradients are torch.clamp's inclusive
// masks on the input values.
//
// Kernel shape (MI355X-first, not the page's Triton tiling):
//   * A group of G lanes owns one row. Lane l handles 16-byte vectors
//     l, l + G, ... of the row, so each wavefront-wide access is 1 KiB
//     contiguous in gate, up, grad_y and the outputs. All V vectors of a pass
//     are loaded (gate, then up, then grad_y) before any math. At inter = 2048
//     the forward spreads a row over 4 wavefronts (1 vector per lane) and the
//     backward over 2 (2 vectors per lane): the shapes that sustained the most
//     bandwidth on MI355X among 1-4 wavefronts per row, 64-1024 thread blocks,
//     persistent grids and register double-buffering across rows.
//   * The probability gradient is a per-lane fp32 register accumulator,
//     reduced with cross-lane shuffles within each wavefront and, when a row
//     spans several wavefronts, through a few LDS slots in a fixed order.
//   * Elementwise streaming work: no MFMA, no LDS tiles, each input byte read
//     once and each output byte written once (nontemporal accesses).
//   * Math per element: compare/select clamps (NaN passes through, as in
//     torch.clamp), exp via v_exp_f32 and 1/(1+e) via v_rcp_f32, the rest
//     fp32 multiplies in the order of the defining expression (built with
//     -ffp-contract=off).
#include "epi_common.h"

namespace moe_epi {
namespace {

// block sizes of the per-element kernels
constexpr int kFwdBlock = 256;
constexpr int kBwdBlock = 128;

// sigma(z) = 1 / (1 + e^-z) with e^-z = 2^(-z * log2(e)).
__device__ __forceinline__ float sigmoid_f32(float z) {
    const float e = __builtin_amdgcn_exp2f(z * -1.4426950408889634f);
    return __builtin_amdgcn_rcpf(1.0f + e);
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

// d_gate, d_up for one element; adds this element's probability-gradient term
// gy * silu(gc) * uc to acc when kGradProbs.
template <bool kGradProbs>
__device__ __forceinline__ void bwd_elem(float g, float u, float gy, float p, float L, float& dg, float& du,
                                         float& acc) {
    const float gc = clamp_hi(g, L);
    const float uc = clamp_sym(u, L);
    const float s = sigmoid_f32(gc);
    const float a = gc * s;  // silu(gc)
    const float t = gy * p;
    if (kGradProbs) acc = __fmaf_rn(gy, a * uc, acc);
    const float dsilu = s * (1.0f + gc * (1.0f - s));
    dg = (g <= L) ? (t * uc) * dsilu : 0.0f;
    du = (fabsf(u) <= L) ? t * a : 0.0f;
}

__device__ __forceinline__ u32x4 fwd_vec(u32x4 g, u32x4 u, float p, float L) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = pack_bf16x2(fwd_elem(bf16_lo(g[i]), bf16_lo(u[i]), p, L), fwd_elem(bf16_hi(g[i]), bf16_hi(u[i]), p, L));
    return o;
}

template <bool kGradProbs>
__device__ __forceinline__ void bwd_vec(u32x4 g, u32x4 u, u32x4 gy, float p, float L, u32x4& dg, u32x4& du,
                                        float& acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float dg0, dg1, du0, du1;
        bwd_elem<kGradProbs>(bf16_lo(g[i]), bf16_lo(u[i]), bf16_lo(gy[i]), p, L, dg0, du0, acc);
        bwd_elem<kGradProbs>(bf16_hi(g[i]), bf16_hi(u[i]), bf16_hi(gy[i]), p, L, dg1, du1, acc);
        dg[i] = pack_bf16x2(dg0, dg1);
        du[i] = pack_bf16x2(du0, du1);
    }
}

// ---- 16-byte vector kernels (inter % 8 == 0, 16-byte aligned tensors) ------
//
// G lanes own a row (G <= 64: part of a wavefront; G = 64*W: W wavefronts),
// B threads per block, B / G rows per block. The row loop advances whole
// blocks, so every thread of a block runs the same iterations (row_sum may
// hold a barrier).

template <int G, int V, int B>
__global__ __launch_bounds__(B) void swiglu_clamped_fwd_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ probs, uint16_t* __restrict__ y, int64_t rows,
    int64_t inter, float L) {
    constexpr int kRows = B / G;
    const int lane = threadIdx.x % G;
    const int64_t nvec = inter / 8;
    for (int64_t rb = static_cast<int64_t>(blockIdx.x) * kRows; rb < rows;
         rb += static_cast<int64_t>(gridDim.x) * kRows) {
        const int64_t r = rb + threadIdx.x / G;
        if (r >= rows) continue;
        const uint16_t* gate = x + r * 2 * inter;
        const uint16_t* up = gate + inter;
        uint16_t* yr = y + r * inter;
        const float p = probs[r];
        for (int64_t c0 = lane; c0 < nvec; c0 += static_cast<int64_t>(G) * V) {
            u32x4 g[V], u[V];
#pragma unroll
            for (int k = 0; k < V; ++k)
                if (c0 + k * G < nvec) g[k] = load_stream(gate + (c0 + k * G) * 8);
#pragma unroll
            for (int k = 0; k < V; ++k)
                if (c0 + k * G < nvec) u[k] = load_stream(up + (c0 + k * G) * 8);
#pragma unroll
            for (int k = 0; k < V; ++k)
                if (c0 + k * G < nvec) store_stream(yr + (c0 + k * G) * 8, fwd_vec(g[k], u[k], p, L));
        }
    }
}

template <int G, int V, int B, bool kGradProbs>
__global__ __launch_bounds__(B) void swiglu_clamped_bwd_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ probs, const uint16_t* __restrict__ grad_y,
    uint16_t* __restrict__ grad_x, float* __restrict__ grad_probs, int64_t rows, int64_t inter, float L) {
    constexpr int kRows = B / G;
    __shared__ float part[B / 64 > 0 ? B / 64 : 1];
    const int lane = threadIdx.x % G;
    const int64_t nvec = inter / 8;
    for (int64_t rb = static_cast<int64_t>(blockIdx.x) * kRows; rb < rows;
         rb += static_cast<int64_t>(gridDim.x) * kRows) {
        const int64_t r = rb + threadIdx.x / G;
        float acc = 0.0f;
        if (r < rows) {
            const uint16_t* gate = x + r * 2 * inter;
            const uint16_t* up = gate + inter;
            const uint16_t* gyr = grad_y + r * inter;
            uint16_t* dgate = grad_x + r * 2 * inter;
            uint16_t* dup = dgate + inter;
            const float p = probs[r];
            for (int64_t c0 = lane; c0 < nvec; c0 += static_cast<int64_t>(G) * V) {
                u32x4 g[V], u[V], gy[V];
#pragma unroll
                for (int k = 0; k < V; ++k)
                    if (c0 + k * G < nvec) g[k] = load_stream(gate + (c0 + k * G) * 8);
#pragma unroll
                for (int k = 0; k < V; ++k)
                    if (c0 + k * G < nvec) u[k] = load_stream(up + (c0 + k * G) * 8);
#pragma unroll
                for (int k = 0; k < V; ++k)
                    if (c0 + k * G < nvec) gy[k] = load_stream(gyr + (c0 + k * G) * 8);
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    if (c0 + k * G < nvec) {
                        u32x4 dg, du;
                        bwd_vec<kGradProbs>(g[k], u[k], gy[k], p, L, dg, du, acc);
                        store_stream(dgate + (c0 + k * G) * 8, dg);
                        store_stream(dup + (c0 + k * G) * 8, du);
                    }
                }
            }
        }
        if constexpr (kGradProbs) {
            acc = row_sum<G>(acc, part);
            if (lane == 0 && r < rows) grad_probs[r] = acc;
        }
    }
}

// ---- per-element kernels (any inter, 2-byte aligned tensors) ---------------

__global__ __launch_bounds__(kFwdBlock) void swiglu_clamped_fwd_scalar_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ probs, uint16_t* __restrict__ y, int64_t rows,
    int64_t inter, float L) {
    constexpr int kRows = kFwdBlock / 64;
    const int lane = threadIdx.x % 64;
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * kRows + threadIdx.x / 64; r < rows;
         r += static_cast<int64_t>(gridDim.x) * kRows) {
        const uint16_t* gate = x + r * 2 * inter;
        const float p = probs[r];
        for (int64_t j = lane; j < inter; j += 64)
            y[r * inter + j] = to_bf16(fwd_elem(bf16_at(gate + j), bf16_at(gate + inter + j), p, L));
    }
}

template <bool kGradProbs>
__global__ __launch_bounds__(kBwdBlock) void swiglu_clamped_bwd_scalar_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ probs, const uint16_t* __restrict__ grad_y,
    uint16_t* __restrict__ grad_x, float* __restrict__ grad_probs, int64_t rows, int64_t inter, float L) {
    constexpr int kRows = kBwdBlock / 64;
    const int lane = threadIdx.x % 64;
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * kRows + threadIdx.x / 64; r < rows;
         r += static_cast<int64_t>(gridDim.x) * kRows) {
        const uint16_t* gate = x + r * 2 * inter;
        uint16_t* dgate = grad_x + r * 2 * inter;
        const float p = probs[r];
        float acc = 0.0f;
        for (int64_t j = lane; j < inter; j += 64) {
            float dg, du;
            bwd_elem<kGradProbs>(bf16_at(gate + j), bf16_at(gate + inter + j), bf16_at(grad_y + r * inter + j), p, L,
                                 dg, du, acc);
            dgate[j] = to_bf16(dg);
            dgate[inter + j] = to_bf16(du);
        }
        if (kGradProbs) {
            acc = group_sum<64>(acc);
            if (lane == 0) grad_probs[r] = acc;
        }
    }
}

// ---- launchers ---------------------------------------------------------------
//
// Shapes (measured on MI355X at 131072 x 2048; nontemporal 16-byte accesses):
//   forward:  one vector per lane (V = 1) and up to 4 wavefronts per row,
//             256-thread blocks (inter = 2048: 4 wavefronts, one row per block);
//   backward: two vectors per lane (V = 2) and as many wavefronts per row as
//             that needs (up to 8), two rows per block (inter = 2048: 2
//             wavefronts per row, 256-thread blocks). Splitting a row over
//             several wavefronts issues its loads from several SIMDs at once;
//             these shapes ran 1-1.5% faster than one wavefront per row.
//   Rows longer than the shape covers take several passes (V is capped).

template <int G, int V, int B>
void launch_fwd(const uint16_t* x, const float* probs, uint16_t* y, int64_t rows, int64_t inter, float L,
                hipStream_t st) {
    hipLaunchKernelGGL((swiglu_clamped_fwd_kernel<G, V, B>), dim3(grid_for_rows(rows, B / G)), dim3(B), 0, st, x,
                       probs, y, rows, inter, L);
}

template <int G, int V, int B>
void launch_bwd(const uint16_t* x, const float* probs, const uint16_t* gy, uint16_t* gx, float* gp, int64_t rows,
                int64_t inter, float L, hipStream_t st) {
    const dim3 grid(grid_for_rows(rows, B / G));
    if (gp)
        hipLaunchKernelGGL((swiglu_clamped_bwd_kernel<G, V, B, true>), grid, dim3(B), 0, st, x, probs, gy, gx, gp,
                           rows, inter, L);
    else
        hipLaunchKernelGGL((swiglu_clamped_bwd_kernel<G, V, B, false>), grid, dim3(B), 0, st, x, probs, gy, gx, gp,
                           rows, inter, L);
}

Shape fwd_shape(int64_t nvec) {
    if (nvec < 64) return Shape{small_group(nvec), 1, 256};
    const int w = pow2_ceil(ceil_div(nvec, 64)) > 4 ? 4 : pow2_ceil(ceil_div(nvec, 64));
    const int64_t v = ceil_div(nvec, 64 * w);
    return Shape{64 * w, static_cast<int>(v > 4 ? 4 : v), 256};
}

Shape bwd_shape(int64_t nvec) {
    if (nvec < 64) return Shape{small_group(nvec), 1, 128};
    if (nvec <= 128) return Shape{64, static_cast<int>(ceil_div(nvec, 64)), 128};
    const int w = pow2_ceil(ceil_div(nvec, 128)) > 8 ? 8 : pow2_ceil(ceil_div(nvec, 128));
    const int64_t v = ceil_div(nvec, 64 * w);
    return Shape{64 * w, static_cast<int>(v > 4 ? 4 : v), 2 * 64 * w > 1024 ? 1024 : 2 * 64 * w};
}

void dispatch_fwd(const uint16_t* x, const float* probs, uint16_t* y, int64_t rows, int64_t inter, float L,
                  hipStream_t st) {
    const Shape sh = fwd_shape(inter / 8);
    switch (sh.G * 8 + sh.V) {
        case 8 * 8 + 1: return launch_fwd<8, 1, 256>(x, probs, y, rows, inter, L, st);
        case 16 * 8 + 1: return launch_fwd<16, 1, 256>(x, probs, y, rows, inter, L, st);
        case 32 * 8 + 1: return launch_fwd<32, 1, 256>(x, probs, y, rows, inter, L, st);
        case 64 * 8 + 1: return launch_fwd<64, 1, 256>(x, probs, y, rows, inter, L, st);
        case 128 * 8 + 1: return launch_fwd<128, 1, 256>(x, probs, y, rows, inter, L, st);
        case 256 * 8 + 1: return launch_fwd<256, 1, 256>(x, probs, y, rows, inter, L, st);
        case 256 * 8 + 2: return launch_fwd<256, 2, 256>(x, probs, y, rows, inter, L, st);
        case 256 * 8 + 3: return launch_fwd<256, 3, 256>(x, probs, y, rows, inter, L, st);
        default: return launch_fwd<256, 4, 256>(x, probs, y, rows, inter, L, st);
    }
}

void dispatch_bwd(const uint16_t* x, const float* probs, const uint16_t* gy, uint16_t* gx, float* gp, int64_t rows,
                  int64_t inter, float L, hipStream_t st) {
    const Shape sh = bwd_shape(inter / 8);
    switch (sh.G * 8 + sh.V) {
        case 8 * 8 + 1: return launch_bwd<8, 1, 128>(x, probs, gy, gx, gp, rows, inter, L, st);
        case 16 * 8 + 1: return launch_bwd<16, 1, 128>(x, probs, gy, gx, gp, rows, inter, L, st);
        case 32 * 8 + 1: return launch_bwd<32, 1, 128>(x, probs, gy, gx, gp, rows, inter, L, st);
        case 64 * 8 + 1: return launch_bwd<64, 1, 128>(x, probs, gy, gx, gp, rows, inter, L, st);
        case 64 * 8 + 2: return launch_bwd<64, 2, 128>(x, probs, gy, gx, gp, rows, inter, L, st);
        case 128 * 8 + 2: return launch_bwd<128, 2, 256>(x, probs, gy, gx, gp, rows, inter, L, st);
        case 256 * 8 + 2: return launch_bwd<256, 2, 512>(x, probs, gy, gx, gp, rows, inter, L, st);
        case 512 * 8 + 2: return launch_bwd<512, 2, 1024>(x, probs, gy, gx, gp, rows, inter, L, st);
        case 512 * 8 + 3: return launch_bwd<512, 3, 1024>(x, probs, gy, gx, gp, rows, inter, L, st);
        default: return launch_bwd<512, 4, 1024>(x, probs, gy, gx, gp, rows, inter, L, st);
    }
}

// Common argument checks; returns MOE_EPI_SUCCESS and fills the byte sizes of
// x / grad_x, of y / grad_y and of probs / grad_probs.
int check_swiglu(int64_t rows, int64_t inter, float limit, int64_t* x_bytes, int64_t* h_bytes, int64_t* p_bytes) {
    if (rows < 0 || inter <= 0 || inter > INT64_MAX / 8) return MOE_EPI_ERR_BAD_SHAPE;
    if (!bytes_ok(rows, 2 * inter, 2, x_bytes) || !bytes_ok(rows, inter, 2, h_bytes) ||
        !bytes_ok(rows, 1, 4, p_bytes))
        return MOE_EPI_ERR_BAD_SHAPE;
    if (!(limit > 0.0f) || !isfinite(limit)) return MOE_EPI_ERR_BAD_LIMIT;
    return MOE_EPI_SUCCESS;
}

}  // namespace
}  // namespace moe_epi

extern "C" int swiglu_clamped_fwd(const uint16_t* x, const float* probs, uint16_t* y, int64_t rows, int64_t inter,
                                  float limit, void* stream) {
    using namespace moe_epi;
    int64_t xb, hb, pb;
    int st = check_swiglu(rows, inter, limit, &xb, &hb, &pb);
    if (st != MOE_EPI_SUCCESS) return st;
    if (rows == 0) return MOE_EPI_SUCCESS;
    if (!x || !probs || !y) return MOE_EPI_ERR_NULL_POINTER;
    if (!aligned(x, 2) || !aligned(y, 2) || !aligned(probs, 4)) return MOE_EPI_ERR_MISALIGNED;
    const Range rx = range_of(x, xb), rp = range_of(probs, pb), ry = range_of(y, hb);
    if (overlaps(ry, rx) || overlaps(ry, rp)) return MOE_EPI_ERR_ALIAS;

    hipStream_t s = as_stream(stream);
    (void)hipGetLastError();
    if (inter % 8 == 0 && aligned(x, 16) && aligned(y, 16)) {
        dispatch_fwd(x, probs, y, rows, inter, limit, s);
    } else {
        hipLaunchKernelGGL(swiglu_clamped_fwd_scalar_kernel, dim3(grid_for_rows(rows, kFwdBlock / 64)),
                           dim3(kFwdBlock), 0, s, x, probs, y, rows, inter, limit);
    }
    return launch_status();
}

extern "C" int swiglu_clamped_bwd(const uint16_t* x, const float* probs, const uint16_t* grad_y, uint16_t* grad_x,
                                  float* grad_probs, int64_t rows, int64_t inter, float limit, void* stream) {
    using namespace moe_epi;
    int64_t xb, hb, pb;
    int st = check_swiglu(rows, inter, limit, &xb, &hb, &pb);
    if (st != MOE_EPI_SUCCESS) return st;
    if (rows == 0) return MOE_EPI_SUCCESS;
    if (!x || !probs || !grad_y || !grad_x) return MOE_EPI_ERR_NULL_POINTER;
    if (!aligned(x, 2) || !aligned(grad_y, 2) || !aligned(grad_x, 2) || !aligned(probs, 4) ||
        (grad_probs && !aligned(grad_probs, 4)))
        return MOE_EPI_ERR_MISALIGNED;
    const Range rx = range_of(x, xb), rp = range_of(probs, pb), rgy = range_of(grad_y, hb);
    const Range rgx = range_of(grad_x, xb), rgp = range_of(grad_probs, grad_probs ? pb : 0);
    if (overlaps(rgx, rx) || overlaps(rgx, rp) || overlaps(rgx, rgy) || overlaps(rgp, rx) || overlaps(rgp, rp) ||
        overlaps(rgp, rgy) || overlaps(rgp, rgx))
        return MOE_EPI_ERR_ALIAS;

    hipStream_t s = as_stream(stream);
    (void)hipGetLastError();
    if (inter % 8 == 0 && aligned(x, 16) && aligned(grad_y, 16) && aligned(grad_x, 16)) {
        dispatch_bwd(x, probs, grad_y, grad_x, grad_probs, rows, inter, limit, s);
    } else {
        const dim3 grid(grid_for_rows(rows, kBwdBlock / 64));
        if (grad_probs)
            hipLaunchKernelGGL(swiglu_clamped_bwd_scalar_kernel<true>, grid, dim3(kBwdBlock), 0, s, x, probs, grad_y,
                               grad_x, grad_probs, rows, inter, limit);
        else
            hipLaunchKernelGGL(swiglu_clamped_bwd_scalar_kernel<false>, grid, dim3(kBwdBlock), 0, s, x, probs,
                               grad_y, grad_x, grad_probs, rows, inter, limit);
    }
    return launch_status();
}
