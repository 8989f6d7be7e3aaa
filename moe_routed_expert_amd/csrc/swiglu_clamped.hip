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
//   * A lane group of G lanes owns one row at a time (G = 64: a whole
//     wavefront per row). Lane l of the group handles vectors l, l + G, ...
//     of the row, each vector being 8 consecutive bf16 columns (16 bytes), so
//     every wavefront-wide access is 1 KiB contiguous for each of gate, up,
//     grad_y and the outputs. V vectors per lane are loaded before any math
//     to keep 2V (forward) or 3V (backward) 16-byte loads in flight per lane.
//   * The probability gradient is a per-lane fp32 register accumulator,
//     reduced across the G lanes with cross-lane shuffles; no LDS.
//   * This is elementwise streaming work: no MFMA, no LDS tiles. Each input
//     byte is read once and each output byte written once.
//   * Math per element: 2 compares/selects for the clamps, exp via v_exp_f32
//     and 1/(1+e) via v_rcp_f32, the rest fp32 multiplies in the same order
//     as the defining expression (built with -ffp-contract=off).
#include "epi_common.h"

namespace moe_epi {
namespace {

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

template <int W, int G, int V>
__global__ __launch_bounds__(kBlock) void swiglu_clamped_fwd_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ probs, uint16_t* __restrict__ y,
    int64_t rows, int64_t inter, float L) {
    constexpr int kGroups = kBlock / G;
    const int lane = threadIdx.x & (G - 1);
    const int64_t nvec = inter / W;
    const int64_t row_step = static_cast<int64_t>(gridDim.x) * kGroups;
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * kGroups + threadIdx.x / G; r < rows; r += row_step) {
        const uint16_t* gate = x + r * 2 * inter;
        const uint16_t* up = gate + inter;
        uint16_t* yr = y + r * inter;
        const float p = probs[r];
        for (int64_t c0 = lane; c0 < nvec; c0 += static_cast<int64_t>(G) * V) {
            float g[V][W], u[V][W];
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const int64_t c = c0 + static_cast<int64_t>(k) * G;
                if (c < nvec) {
                    Io<W>::load(gate + c * W, g[k]);
                    Io<W>::load(up + c * W, u[k]);
                }
            }
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const int64_t c = c0 + static_cast<int64_t>(k) * G;
                if (c < nvec) {
                    float o[W];
#pragma unroll
                    for (int e = 0; e < W; ++e) {
                        const float gc = clamp_hi(g[k][e], L);
                        const float uc = clamp_sym(u[k][e], L);
                        const float s = sigmoid_f32(gc);
                        o[e] = ((gc * s) * uc) * p;
                    }
                    Io<W>::store(yr + c * W, o);
                }
            }
        }
    }
}

template <int W, int G, int V, bool kGradProbs>
__global__ __launch_bounds__(kBlock) void swiglu_clamped_bwd_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ probs, const uint16_t* __restrict__ grad_y,
    uint16_t* __restrict__ grad_x, float* __restrict__ grad_probs, int64_t rows, int64_t inter, float L) {
    constexpr int kGroups = kBlock / G;
    const int lane = threadIdx.x & (G - 1);
    const int64_t nvec = inter / W;
    const int64_t row_step = static_cast<int64_t>(gridDim.x) * kGroups;
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * kGroups + threadIdx.x / G; r < rows; r += row_step) {
        const uint16_t* gate = x + r * 2 * inter;
        const uint16_t* up = gate + inter;
        const uint16_t* gyr = grad_y + r * inter;
        uint16_t* dgate = grad_x + r * 2 * inter;
        uint16_t* dup = dgate + inter;
        const float p = probs[r];
        float acc = 0.0f;
        for (int64_t c0 = lane; c0 < nvec; c0 += static_cast<int64_t>(G) * V) {
            float g[V][W], u[V][W], gy[V][W];
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const int64_t c = c0 + static_cast<int64_t>(k) * G;
                if (c < nvec) {
                    Io<W>::load(gate + c * W, g[k]);
                    Io<W>::load(up + c * W, u[k]);
                    Io<W>::load(gyr + c * W, gy[k]);
                }
            }
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const int64_t c = c0 + static_cast<int64_t>(k) * G;
                if (c < nvec) {
                    float dg[W], du[W];
#pragma unroll
                    for (int e = 0; e < W; ++e) {
                        const float gv = g[k][e], uv = u[k][e];
                        const float gc = clamp_hi(gv, L);
                        const float uc = clamp_sym(uv, L);
                        const float s = sigmoid_f32(gc);
                        const float a = gc * s;                 // silu(gc)
                        const float t = gy[k][e] * p;
                        if (kGradProbs) acc = __fmaf_rn(gy[k][e], a * uc, acc);
                        const float dsilu = s * (1.0f + gc * (1.0f - s));
                        dg[e] = (gv <= L) ? (t * uc) * dsilu : 0.0f;
                        du[e] = (fabsf(uv) <= L) ? t * a : 0.0f;
                    }
                    Io<W>::store(dgate + c * W, dg);
                    Io<W>::store(dup + c * W, du);
                }
            }
        }
        if (kGradProbs) {
            acc = group_sum<G>(acc);
            if (lane == 0) grad_probs[r] = acc;
        }
    }
}

// Lane-group width G and vectors per lane V for a row of nvec vectors.
struct Shape {
    int G, V;
};

inline Shape pick_shape(int64_t nvec) {
    if (nvec >= 64) {
        int64_t v = (nvec + 63) / 64;
        return Shape{64, static_cast<int>(v > 4 ? 4 : v)};
    }
    if (nvec > 16) return Shape{32, 1};
    if (nvec > 8) return Shape{16, 1};
    return Shape{8, 1};
}

constexpr int64_t kMaxBlocks = 1 << 20;  // 2^28 work-items at most; the row loop strides over the rest

template <int W, int G, int V>
void launch_fwd(const uint16_t* x, const float* probs, uint16_t* y, int64_t rows, int64_t inter, float L,
                hipStream_t st) {
    const unsigned grid = grid_for_rows(rows, kBlock / G, kMaxBlocks);
    hipLaunchKernelGGL((swiglu_clamped_fwd_kernel<W, G, V>), dim3(grid), dim3(kBlock), 0, st, x, probs, y, rows,
                       inter, L);
}

template <int W, int G, int V>
void launch_bwd(const uint16_t* x, const float* probs, const uint16_t* gy, uint16_t* gx, float* gp, int64_t rows,
                int64_t inter, float L, hipStream_t st) {
    const unsigned grid = grid_for_rows(rows, kBlock / G, kMaxBlocks);
    if (gp)
        hipLaunchKernelGGL((swiglu_clamped_bwd_kernel<W, G, V, true>), dim3(grid), dim3(kBlock), 0, st, x, probs, gy,
                           gx, gp, rows, inter, L);
    else
        hipLaunchKernelGGL((swiglu_clamped_bwd_kernel<W, G, V, false>), dim3(grid), dim3(kBlock), 0, st, x, probs,
                           gy, gx, gp, rows, inter, L);
}

#define MOE_EPI_DISPATCH_SHAPE(SHAPE, LAUNCH, ...)                          \
    do {                                                                    \
        if ((SHAPE).G == 64 && (SHAPE).V == 4) LAUNCH<8, 64, 4>(__VA_ARGS__); \
        else if ((SHAPE).G == 64 && (SHAPE).V == 3) LAUNCH<8, 64, 3>(__VA_ARGS__); \
        else if ((SHAPE).G == 64 && (SHAPE).V == 2) LAUNCH<8, 64, 2>(__VA_ARGS__); \
        else if ((SHAPE).G == 64) LAUNCH<8, 64, 1>(__VA_ARGS__);            \
        else if ((SHAPE).G == 32) LAUNCH<8, 32, 1>(__VA_ARGS__);            \
        else if ((SHAPE).G == 16) LAUNCH<8, 16, 1>(__VA_ARGS__);            \
        else LAUNCH<8, 8, 1>(__VA_ARGS__);                                  \
    } while (0)

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
        const Shape sh = pick_shape(inter / 8);
        MOE_EPI_DISPATCH_SHAPE(sh, launch_fwd, x, probs, y, rows, inter, limit, s);
    } else {
        launch_fwd<1, 64, 4>(x, probs, y, rows, inter, limit, s);
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
        const Shape sh = pick_shape(inter / 8);
        MOE_EPI_DISPATCH_SHAPE(sh, launch_bwd, x, probs, grad_y, grad_x, grad_probs, rows, inter, limit, s);
    } else {
        launch_bwd<1, 64, 4>(x, probs, grad_y, grad_x, grad_probs, rows, inter, limit, s);
    }
    return launch_status();
}
