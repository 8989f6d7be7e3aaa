// Clamped SwiGLU times routing probability: forward and single-pass backward
// for gfx950.
//
// Operation (page "nemo_automodel.components.moe.swiglu_triton", module
// description): on the grouped-GEMM output x = [gate | up] ([rows, 2*inter],
// bf16, fp16 or fp32) with one fp32 probability per row,
//   y = silu(min(gate, L)) * clamp(up, -L, L) * p,
// computed in fp32 and rounded once to x's dtype. The backward writes d_gate
// and d_up into the two halves of grad_x and reduces the per-row probability
// gradient in registers; its clamp gradients follow torch.clamp (masks on the
// input values, bounds included).
//
// Kernel shape (MI355X-first, not the page's Triton tiling):
//   * A group of G lanes owns one row. Lane l handles vectors of 8 elements
//     l, l + G, ... of the row (16 bytes for 16-bit types), so each
//     wavefront-wide access is 1 KiB contiguous in gate, up, grad_y and the
//     outputs. All V vectors of a pass are loaded (gate, then up, then grad_y)
//     before any math. At inter = 2048 (256 vectors) both kernels spread a row
//     over 3 wavefronts (192 lanes: the first wavefront takes vectors 0-63
//     and 192-255, the other two one vector per lane; the backward loads the
//     first wavefront's two vectors together) and put three rows in a
//     576-lane block: the shapes that sustained the most bandwidth on MI355X,
//     with the caches flushed before every launch, among 1-4 wavefronts per
//     row, 1-5 rows per block, 64-1024 thread blocks, block orders that give
//     each XCD contiguous runs of rows, persistent grids and register
//     double-buffering across rows (the launchers below give the measured
//     alternatives).
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
#include "swiglu_math.h"

namespace moe_epi {
namespace {

// block sizes of the per-element kernels
constexpr int kFwdBlock = 256;
constexpr int kBwdBlock = 128;

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

template <int T>
__device__ __forceinline__ typename Elem<T>::Raw fwd_vec(typename Elem<T>::Raw g, typename Elem<T>::Raw u, float p,
                                                         float L) {
    float gf[8], uf[8], o[8];
    Elem<T>::unpack(g, gf);
    Elem<T>::unpack(u, uf);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = fwd_elem(gf[e], uf[e], p, L);
    return Elem<T>::pack(o);
}

template <int T, bool kGradProbs>
__device__ __forceinline__ void bwd_vec(typename Elem<T>::Raw g, typename Elem<T>::Raw u, typename Elem<T>::Raw gy,
                                        float p, float L, typename Elem<T>::Raw& dg, typename Elem<T>::Raw& du,
                                        float& acc) {
    float gf[8], uf[8], yf[8], dgf[8], duf[8];
    Elem<T>::unpack(g, gf);
    Elem<T>::unpack(u, uf);
    Elem<T>::unpack(gy, yf);
#pragma unroll
    for (int e = 0; e < 8; ++e) bwd_elem<kGradProbs>(gf[e], uf[e], yf[e], p, L, dgf[e], duf[e], acc);
    dg = Elem<T>::pack(dgf);
    du = Elem<T>::pack(duf);
}

// ---- vector kernels (inter % 8 == 0, 16-byte aligned tensors) ---------------
//
// G lanes own a row (G <= 64: part of a wavefront; G = 64*W: W wavefronts),
// B threads per block, B / G rows per block. The row loop advances whole
// blocks, so every thread of a block runs the same iterations (row_sum may
// hold a barrier). Element offsets below are in elements of T.

// kAlign: the block's wavefronts meet at a barrier before any of them issues
// its row loads (align_block_loads, epi_common.h).
template <int T, int G, int V, int B, bool kAlign>
__global__ __launch_bounds__(B) void swiglu_clamped_fwd_kernel(const void* __restrict__ x,
                                                               const float* __restrict__ probs, void* __restrict__ y,
                                                               int64_t rows, int64_t inter, float L) {
    using E = Elem<T>;
    constexpr bool kSplit = T == MOE_EPI_F32;  // the vector map (epi_common.h)
    constexpr int kRows = B / G;
    const uint32_t lane = threadIdx.x % G;
    const uint32_t nvec = static_cast<uint32_t>(inter / 8);
    for (int64_t rb = static_cast<int64_t>(blockIdx.x) * kRows; rb < rows;
         rb += static_cast<int64_t>(gridDim.x) * kRows) {
        const int64_t r = rb + group_in_block<G>();
        const float p = r < rows ? probs[r] : 0.0f;
        if constexpr (kAlign) align_block_loads();
        if (r >= rows) continue;
        const void* xg = row_at<T>(x, r * 2 * inter);
        const void* xu = row_at<T>(x, r * 2 * inter + inter);
        void* yr = row_at<T>(y, r * inter);
        for (uint32_t c0 = lane; c0 < nvec; c0 += G * V) {
            typename E::Raw g[V], u[V];
            Quads q[V];
#pragma unroll
            for (int k = 0; k < V; ++k) q[k] = quads_of<G, kSplit>(c0 + k * G, lane, nvec);
#pragma unroll
            for (int k = 0; k < V; ++k)
                if (c0 + k * G < nvec) g[k] = E::template load<kSplit>(xg, q[k]);
#pragma unroll
            for (int k = 0; k < V; ++k)
                if (c0 + k * G < nvec) u[k] = E::template load<kSplit>(xu, q[k]);
#pragma unroll
            for (int k = 0; k < V; ++k)
                if (c0 + k * G < nvec) E::template store<kSplit>(yr, q[k], fwd_vec<T>(g[k], u[k], p, L));
        }
    }
}

template <int T, int G, int V, int B, bool kGradProbs, bool kAlign>
__global__ __launch_bounds__(B) __attribute__((amdgpu_waves_per_eu(waves_for_two_blocks(B)))) void
swiglu_clamped_bwd_kernel(const void* __restrict__ x, const float* __restrict__ probs, const void* __restrict__ grad_y,
                          void* __restrict__ grad_x, float* __restrict__ grad_probs, int64_t rows, int64_t inter,
                          float L) {
    using E = Elem<T>;
    constexpr bool kSplit = T == MOE_EPI_F32;  // the vector map (epi_common.h)
    constexpr int kRows = B / G;
    __shared__ float part[B / 64 > 0 ? B / 64 : 1];
    const uint32_t lane = threadIdx.x % G;
    const uint32_t nvec = static_cast<uint32_t>(inter / 8);
    for (int64_t rb = static_cast<int64_t>(blockIdx.x) * kRows; rb < rows;
         rb += static_cast<int64_t>(gridDim.x) * kRows) {
        const int64_t r = rb + group_in_block<G>();
        float acc = 0.0f;
        const float p = r < rows ? probs[r] : 0.0f;
        if constexpr (kAlign) align_block_loads();
        if (r < rows) {
            const void* xg = row_at<T>(x, r * 2 * inter);
            const void* xu = row_at<T>(x, r * 2 * inter + inter);
            const void* gyr = row_at<T>(grad_y, r * inter);
            void* gxg = row_at<T>(grad_x, r * 2 * inter);
            void* gxu = row_at<T>(grad_x, r * 2 * inter + inter);
            for (uint32_t c0 = lane; c0 < nvec; c0 += G * V) {
                typename E::Raw g[V], u[V], gy[V];
                Quads q[V];
#pragma unroll
                for (int k = 0; k < V; ++k) q[k] = quads_of<G, kSplit>(c0 + k * G, lane, nvec);
#pragma unroll
                for (int k = 0; k < V; ++k)
                    if (c0 + k * G < nvec) g[k] = E::template load<kSplit>(xg, q[k]);
#pragma unroll
                for (int k = 0; k < V; ++k)
                    if (c0 + k * G < nvec) u[k] = E::template load<kSplit>(xu, q[k]);
#pragma unroll
                for (int k = 0; k < V; ++k)
                    if (c0 + k * G < nvec) gy[k] = E::template load<kSplit>(gyr, q[k]);
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    if (c0 + k * G < nvec) {
                        typename E::Raw dg, du;
                        bwd_vec<T, kGradProbs>(g[k], u[k], gy[k], p, L, dg, du, acc);
                        E::template store<kSplit>(gxg, q[k], dg);
                        E::template store<kSplit>(gxu, q[k], du);
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

// ---- per-element kernels (any inter, element-aligned tensors) ---------------

template <int T>
__global__ __launch_bounds__(kFwdBlock) void swiglu_clamped_fwd_scalar_kernel(const void* __restrict__ x,
                                                                              const float* __restrict__ probs,
                                                                              void* __restrict__ y, int64_t rows,
                                                                              int64_t inter, float L) {
    using E = Elem<T>;
    constexpr int kRows = kFwdBlock / 64;
    const int lane = threadIdx.x % 64;
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * kRows + threadIdx.x / 64; r < rows;
         r += static_cast<int64_t>(gridDim.x) * kRows) {
        const int64_t gate = r * 2 * inter;
        const float p = probs[r];
        for (int64_t j = lane; j < inter; j += 64)
            E::store1(y, r * inter + j, fwd_elem(E::load1(x, gate + j), E::load1(x, gate + inter + j), p, L));
    }
}

template <int T, bool kGradProbs>
__global__ __launch_bounds__(kBwdBlock) void swiglu_clamped_bwd_scalar_kernel(
    const void* __restrict__ x, const float* __restrict__ probs, const void* __restrict__ grad_y,
    void* __restrict__ grad_x, float* __restrict__ grad_probs, int64_t rows, int64_t inter, float L) {
    using E = Elem<T>;
    constexpr int kRows = kBwdBlock / 64;
    const int lane = threadIdx.x % 64;
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * kRows + threadIdx.x / 64; r < rows;
         r += static_cast<int64_t>(gridDim.x) * kRows) {
        const int64_t gate = r * 2 * inter;
        const float p = probs[r];
        float acc = 0.0f;
        for (int64_t j = lane; j < inter; j += 64) {
            float dg, du;
            bwd_elem<kGradProbs>(E::load1(x, gate + j), E::load1(x, gate + inter + j), E::load1(grad_y, r * inter + j),
                                 p, L, dg, du, acc);
            E::store1(grad_x, gate + j, dg);
            E::store1(grad_x, gate + inter + j, du);
        }
        if (kGradProbs) {
            acc = group_sum<64>(acc);
            if (lane == 0) grad_probs[r] = acc;
        }
    }
}

// ---- launchers ---------------------------------------------------------------
//
// Launch shapes: G lanes per row, V vectors per lane per pass, B threads per
// block (B / G rows per block). For rows of 192 vectors (1536 columns) and
// more they come from a sweep on MI355X of 59 forward and 40 backward shapes
// per dtype at 1536, 2048, 4096 and 8192 columns (100003, 131072, 65536 and
// 32768 rows), one table per element width: each entry is the shape whose
// worst case over the dtypes sharing it was best, and every entry was within
// 2.5% of that case's fastest shape (the shapes they replace lost up to 16%).
// What the sweep showed:
//  - one row per block beats two in the backward (the row sum's barrier then
//    holds only that row's waves);
//  - the best shapes keep few rows in flight per CU, each streamed by many
//    wavefronts, even where that leaves lanes idle (448 lanes for 192 float32
//    vectors): fewer, longer runs per DRAM page;
//  - float32 wants more lanes per row than 16-bit types at the same width.
// Narrower rows keep the earlier rules (a wavefront or less per row for
// under 64 vectors, up to 4 wavefronts between 64 and 191). Rows wider than a
// shape covers take several passes.

template <int T, int G, int V, int B, bool kAlign = false>
void launch_fwd(const void* x, const float* probs, void* y, int64_t rows, int64_t inter, float L, hipStream_t st) {
    hipLaunchKernelGGL((swiglu_clamped_fwd_kernel<T, G, V, B, kAlign>), dim3(grid_for_rows(rows, B / G)), dim3(B), 0,
                       st, x, probs, y, rows, inter, L);
}

template <int T, int G, int V, int B, bool kAlign = false>
void launch_bwd(const void* x, const float* probs, const void* gy, void* gx, float* gp, int64_t rows, int64_t inter,
                float L, hipStream_t st) {
    const dim3 grid(grid_for_rows(rows, B / G));
    if (gp)
        hipLaunchKernelGGL((swiglu_clamped_bwd_kernel<T, G, V, B, true, kAlign>), grid, dim3(B), 0, st, x, probs, gy, gx,
                           gp, rows, inter, L);
    else
        hipLaunchKernelGGL((swiglu_clamped_bwd_kernel<T, G, V, B, false, kAlign>), grid, dim3(B), 0, st, x, probs, gy,
                           gx, gp, rows, inter, L);
}

// Up to this many rows (64 per CU on the 256-CU part) a launch is short
// enough that its ramp and tail weigh more than the steady stream: one row per
// block, unaligned, spreads the last blocks better. bfloat16 at inter 2048,
// caches flushed: 8192 rows, forward 61.2% of HBM peak against 58.6% for three
// aligned 192-lane rows per block, backward 66.3% against 61.6%; 16384 rows,
// 70.9 / 73.3% against 70.1 / 71.9%; 32768 rows even; 65536 rows and above
// the three aligned rows lead by 3-4 points.
constexpr int64_t kFewRows = 16384;

template <int T>
void dispatch_fwd(const void* x, const float* probs, void* y, int64_t rows, int64_t inter, float L, hipStream_t st) {
    const int64_t nvec = inter / 8;
    if (nvec < 64) {
        switch (small_group(nvec)) {
            case 8: return launch_fwd<T, 8, 1, 256>(x, probs, y, rows, inter, L, st);
            case 16: return launch_fwd<T, 16, 1, 256>(x, probs, y, rows, inter, L, st);
            default: return launch_fwd<T, 32, 1, 256>(x, probs, y, rows, inter, L, st);
        }
    }
    if (nvec == 64) return launch_fwd<T, 64, 1, 256>(x, probs, y, rows, inter, L, st);
    if (nvec <= 128) return launch_fwd<T, 128, 1, 256>(x, probs, y, rows, inter, L, st);
    if (nvec < 192) return launch_fwd<T, 256, 1, 256>(x, probs, y, rows, inter, L, st);
    // At the widths of the workloads (192 and 256 vectors) the shapes come from
    // a second sweep, per dtype, with the option of aligned row loads
    // (align_block_loads, epi_common.h): the alignment helped bfloat16 and
    // float32 and hurt float16 there, so each choice below holds only for the
    // dtype it was measured on.
    if constexpr (T == MOE_EPI_F32) {
        // 256 vectors, aligned: 86.0% of HBM peak against 78.3% unaligned
        if (nvec == 256) return launch_fwd<T, 448, 4, 448, true>(x, probs, y, rows, inter, L, st);
        if (nvec <= 512) return launch_fwd<T, 448, 4, 448>(x, probs, y, rows, inter, L, st);
        return launch_fwd<T, 384, 1, 384>(x, probs, y, rows, inter, L, st);
    } else {
        // 192 vectors (inter 1536), bfloat16: 128 lanes per row (the first
        // wavefront takes two vectors per lane), three rows per block,
        // aligned: 81.2% of HBM peak against 79.5% for two unaligned 256-lane
        // rows per block (the shape float16 keeps)
        if (nvec == 192) {
            if constexpr (T == MOE_EPI_BF16) return launch_fwd<T, 128, 1, 384, true>(x, probs, y, rows, inter, L, st);
            return launch_fwd<T, 256, 1, 512>(x, probs, y, rows, inter, L, st);
        }
        // a full 256-vector row (inter 2048): 192 lanes per row (the first
        // wavefront takes vectors 0-63 and 192-255, the others one vector per
        // lane), three rows per 576-lane block. bfloat16 with the block aligned
        // before its loads: 85.1-85.5% of HBM peak (caches flushed before every
        // launch), against 80.8-81.0% for the same shape unaligned, 79.8-80.6%
        // for four 256-lane rows per 1024-lane block (aligned or not), 83.7-84.2%
        // for two aligned 192-lane rows. float16 unaligned: 85.0%, against
        // 82.9% aligned and 77.7% for four 256-lane rows.
        if (nvec == 256) {
            if constexpr (T == MOE_EPI_BF16) {
                if (rows <= kFewRows) return launch_fwd<T, 128, 2, 256>(x, probs, y, rows, inter, L, st);
                return launch_fwd<T, 192, 1, 576, true>(x, probs, y, rows, inter, L, st);
            }
            return launch_fwd<T, 192, 1, 576>(x, probs, y, rows, inter, L, st);
        }
        // 193-255 vectors: 192 lanes per row, two rows per block (224 vectors: 82.4%
        // against 79.7% for 256 lanes, one row; 193 vectors: the same within 0.5%)
        if (nvec < 256) return launch_fwd<T, 192, 1, 384>(x, probs, y, rows, inter, L, st);
        return launch_fwd<T, 1024, 1, 1024>(x, probs, y, rows, inter, L, st);
    }
}

template <int T>
void dispatch_bwd(const void* x, const float* probs, const void* gy, void* gx, float* gp, int64_t rows, int64_t inter,
                  float L, hipStream_t st) {
    const int64_t nvec = inter / 8;
    if (nvec < 64) {
        switch (small_group(nvec)) {
            case 8: return launch_bwd<T, 8, 1, 128>(x, probs, gy, gx, gp, rows, inter, L, st);
            case 16: return launch_bwd<T, 16, 1, 128>(x, probs, gy, gx, gp, rows, inter, L, st);
            default: return launch_bwd<T, 32, 1, 128>(x, probs, gy, gx, gp, rows, inter, L, st);
        }
    }
    if (nvec == 64) return launch_bwd<T, 64, 1, 128>(x, probs, gy, gx, gp, rows, inter, L, st);
    if (nvec <= 128) return launch_bwd<T, 64, 2, 128>(x, probs, gy, gx, gp, rows, inter, L, st);
    if (nvec < 192) return launch_bwd<T, 128, 2, 256>(x, probs, gy, gx, gp, rows, inter, L, st);
    if constexpr (T == MOE_EPI_F32) {
        // 256 vectors, aligned: 81.9% of HBM peak against 79.4% unaligned
        if (nvec == 256) return launch_bwd<T, 384, 2, 384, true>(x, probs, gy, gx, gp, rows, inter, L, st);
        if (nvec <= 256) return launch_bwd<T, 384, 2, 384>(x, probs, gy, gx, gp, rows, inter, L, st);
        if (nvec <= 512) return launch_bwd<T, 640, 2, 640>(x, probs, gy, gx, gp, rows, inter, L, st);
        return launch_bwd<T, 512, 1, 1024>(x, probs, gy, gx, gp, rows, inter, L, st);
    } else {
        // 192 vectors (inter 1536), bfloat16: one vector per lane of 192, three
        // rows per block, aligned: 82.2% of HBM peak against 78.3% for two
        // unaligned 256-lane rows per block (the shape float16 keeps)
        if (nvec == 192) {
            if constexpr (T == MOE_EPI_BF16)
                return launch_bwd<T, 192, 1, 576, true>(x, probs, gy, gx, gp, rows, inter, L, st);
            return launch_bwd<T, 256, 1, 512>(x, probs, gy, gx, gp, rows, inter, L, st);
        }
        // 256 vectors (inter 2048): three 192-lane rows per block. bfloat16
        // aligned before the loads: 82.8-83.1% of HBM peak, against 78.6%
        // unaligned, 81.1-82.0% with the first wavefront's two vectors loaded
        // together, 79.6-80.5% for two 192-lane rows (aligned or not); without
        // the probability gradient the same shape (81.1%; 81.4% for two
        // 512-lane rows). float16, unaligned: two 192-lane rows per block,
        // 82.3-82.7% against 81.0-81.3% for three; without the probability
        // gradient two 512-lane rows (half the lanes idle, no row reduction):
        // 82.2-82.5% against 77.4-77.7% for three 192-lane rows (with the
        // reduction that shape falls to 70.4%).
        if (nvec == 256) {
            if constexpr (T == MOE_EPI_BF16) {
                if (rows <= kFewRows) return launch_bwd<T, 256, 1, 256>(x, probs, gy, gx, gp, rows, inter, L, st);
                return launch_bwd<T, 192, 1, 576, true>(x, probs, gy, gx, gp, rows, inter, L, st);
            }
            if (!gp) return launch_bwd<T, 512, 1, 1024>(x, probs, gy, gx, gp, rows, inter, L, st);
            return launch_bwd<T, 192, 1, 384>(x, probs, gy, gx, gp, rows, inter, L, st);
        }
        if (nvec <= 256) return launch_bwd<T, 192, 1, 384>(x, probs, gy, gx, gp, rows, inter, L, st);
        if (nvec <= 512) return launch_bwd<T, 448, 1, 448>(x, probs, gy, gx, gp, rows, inter, L, st);
        return launch_bwd<T, 512, 2, 512>(x, probs, gy, gx, gp, rows, inter, L, st);
    }
}

template <int T>
void run_fwd(const void* x, const float* probs, void* y, int64_t rows, int64_t inter, float L, bool vec,
             hipStream_t st) {
    if (vec)
        dispatch_fwd<T>(x, probs, y, rows, inter, L, st);
    else
        hipLaunchKernelGGL((swiglu_clamped_fwd_scalar_kernel<T>), dim3(grid_for_rows(rows, kFwdBlock / 64)),
                           dim3(kFwdBlock), 0, st, x, probs, y, rows, inter, L);
}

template <int T>
void run_bwd(const void* x, const float* probs, const void* gy, void* gx, float* gp, int64_t rows, int64_t inter,
             float L, bool vec, hipStream_t st) {
    if (vec) {
        dispatch_bwd<T>(x, probs, gy, gx, gp, rows, inter, L, st);
        return;
    }
    const dim3 grid(grid_for_rows(rows, kBwdBlock / 64));
    if (gp)
        hipLaunchKernelGGL((swiglu_clamped_bwd_scalar_kernel<T, true>), grid, dim3(kBwdBlock), 0, st, x, probs, gy, gx,
                           gp, rows, inter, L);
    else
        hipLaunchKernelGGL((swiglu_clamped_bwd_scalar_kernel<T, false>), grid, dim3(kBwdBlock), 0, st, x, probs, gy,
                           gx, gp, rows, inter, L);
}

// Common argument checks; returns MOE_EPI_SUCCESS and fills the byte sizes of
// x / grad_x, of y / grad_y and of probs / grad_probs.
int check_swiglu(int64_t rows, int64_t inter, float limit, int dtype, int64_t* x_bytes, int64_t* h_bytes,
                 int64_t* p_bytes) {
    if (!dtype_ok(dtype)) return MOE_EPI_ERR_BAD_DTYPE;
    if (rows < 0 || inter <= 0 || inter > INT64_MAX / 8) return MOE_EPI_ERR_BAD_SHAPE;
    const int eb = elem_bytes(dtype);
    if (!bytes_ok(rows, 2 * inter, eb, x_bytes) || !bytes_ok(rows, inter, eb, h_bytes) ||
        !bytes_ok(rows, 1, 4, p_bytes))
        return MOE_EPI_ERR_BAD_SHAPE;
    if (!(limit > 0.0f) || !isfinite(limit)) return MOE_EPI_ERR_BAD_LIMIT;
    return MOE_EPI_SUCCESS;
}

int swiglu_fwd_impl(const void* x, const float* probs, void* y, int64_t rows, int64_t inter, float limit, int dtype,
                    void* stream) {
    int64_t xb, hb, pb;
    int st = check_swiglu(rows, inter, limit, dtype, &xb, &hb, &pb);
    if (st != MOE_EPI_SUCCESS) return st;
    if (rows == 0) return MOE_EPI_SUCCESS;
    if (!x || !probs || !y) return MOE_EPI_ERR_NULL_POINTER;
    const int eb = elem_bytes(dtype);
    if (!aligned(x, eb) || !aligned(y, eb) || !aligned(probs, 4)) return MOE_EPI_ERR_MISALIGNED;
    const Range rx = range_of(x, xb), rp = range_of(probs, pb), ry = range_of(y, hb);
    if (overlaps(ry, rx) || overlaps(ry, rp)) return MOE_EPI_ERR_ALIAS;

    hipStream_t s = as_stream(stream);
    (void)hipGetLastError();
    const bool vec = inter % 8 == 0 && row_fits_u32_offsets(2 * inter, eb) && aligned(x, 16) && aligned(y, 16);
    switch (dtype) {
        case MOE_EPI_BF16: run_fwd<MOE_EPI_BF16>(x, probs, y, rows, inter, limit, vec, s); break;
        case MOE_EPI_F16: run_fwd<MOE_EPI_F16>(x, probs, y, rows, inter, limit, vec, s); break;
        default: run_fwd<MOE_EPI_F32>(x, probs, y, rows, inter, limit, vec, s); break;
    }
    return launch_status();
}

int swiglu_bwd_impl(const void* x, const float* probs, const void* grad_y, void* grad_x, float* grad_probs,
                    int64_t rows, int64_t inter, float limit, int dtype, void* stream) {
    int64_t xb, hb, pb;
    int st = check_swiglu(rows, inter, limit, dtype, &xb, &hb, &pb);
    if (st != MOE_EPI_SUCCESS) return st;
    if (rows == 0) return MOE_EPI_SUCCESS;
    if (!x || !probs || !grad_y || !grad_x) return MOE_EPI_ERR_NULL_POINTER;
    const int eb = elem_bytes(dtype);
    if (!aligned(x, eb) || !aligned(grad_y, eb) || !aligned(grad_x, eb) || !aligned(probs, 4) ||
        (grad_probs && !aligned(grad_probs, 4)))
        return MOE_EPI_ERR_MISALIGNED;
    const Range rx = range_of(x, xb), rp = range_of(probs, pb), rgy = range_of(grad_y, hb);
    const Range rgx = range_of(grad_x, xb), rgp = range_of(grad_probs, grad_probs ? pb : 0);
    if (overlaps(rgx, rx) || overlaps(rgx, rp) || overlaps(rgx, rgy) || overlaps(rgp, rx) || overlaps(rgp, rp) ||
        overlaps(rgp, rgy) || overlaps(rgp, rgx))
        return MOE_EPI_ERR_ALIAS;

    hipStream_t s = as_stream(stream);
    (void)hipGetLastError();
    const bool vec = inter % 8 == 0 && row_fits_u32_offsets(2 * inter, eb) && aligned(x, 16) && aligned(grad_y, 16) &&
                     aligned(grad_x, 16);
    switch (dtype) {
        case MOE_EPI_BF16: run_bwd<MOE_EPI_BF16>(x, probs, grad_y, grad_x, grad_probs, rows, inter, limit, vec, s); break;
        case MOE_EPI_F16: run_bwd<MOE_EPI_F16>(x, probs, grad_y, grad_x, grad_probs, rows, inter, limit, vec, s); break;
        default: run_bwd<MOE_EPI_F32>(x, probs, grad_y, grad_x, grad_probs, rows, inter, limit, vec, s); break;
    }
    return launch_status();
}

}  // namespace
}  // namespace moe_epi

extern "C" int swiglu_clamped_fwd(const uint16_t* x, const float* probs, uint16_t* y, int64_t rows, int64_t inter,
                                  float limit, void* stream) {
    return moe_epi::swiglu_fwd_impl(x, probs, y, rows, inter, limit, MOE_EPI_BF16, stream);
}

extern "C" int swiglu_clamped_bwd(const uint16_t* x, const float* probs, const uint16_t* grad_y, uint16_t* grad_x,
                                  float* grad_probs, int64_t rows, int64_t inter, float limit, void* stream) {
    return moe_epi::swiglu_bwd_impl(x, probs, grad_y, grad_x, grad_probs, rows, inter, limit, MOE_EPI_BF16, stream);
}

extern "C" int swiglu_clamped_fwd_typed(const void* x, const float* probs, void* y, int64_t rows, int64_t inter,
                                        float limit, int dtype, void* stream) {
    return moe_epi::swiglu_fwd_impl(x, probs, y, rows, inter, limit, dtype, stream);
}

extern "C" int swiglu_clamped_bwd_typed(const void* x, const float* probs, const void* grad_y, void* grad_x,
                                        float* grad_probs, int64_t rows, int64_t inter, float limit, int dtype,
                                        void* stream) {
    return moe_epi::swiglu_bwd_impl(x, probs, grad_y, grad_x, grad_probs, rows, inter, limit, dtype, stream);
}
