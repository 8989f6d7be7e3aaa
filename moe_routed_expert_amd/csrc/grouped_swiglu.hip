// gate_up grouped GEMM with the clamped SwiGLU x probability epilogue, for
// gfx950 (bf16 MFMA, fp32 accumulation).
//
// Operation. Pages: "nemo_automodel.components.moe.mok_experts" (the routed
// gate and up weights are contiguous bf16 [local_experts,
// expert_intermediate, hidden]); "nemo_automodel.components.moe.
// quantized_experts", MXFP4ExpertStorageMixin._mxfp4_base_mm (the routed
// activations are [tokens, in_dim], grouped contiguously by local expert;
// offs is an int32 [local_experts] tensor of cumulative token counts; the
// product is [tokens, out_dim] in the activation dtype);
// "nemo_automodel.components.moe.swiglu_triton" (the clamped SwiGLU epilogue
// applied to that grouped-GEMM output x = [gate | up]). For a row t of local
// expert e, rows [start_e, end_e) with start_0 = 0 and end_e = offs[e]
// clamped to [start_e, tokens]:
//   gate[t, j] = bf16(sum_h a[t, h] * w_gate[e, j, h])   (fp32 accumulation)
//   up[t, j]   = bf16(sum_h a[t, h] * w_up[e, j, h])
//   y[t, j]    = bf16(silu(min(gate, L)) * clamp(up, -L, L) * p[t])
// with the epilogue computed from the bf16 gate and up, exactly as the
// streaming forward computes it from a stored x. x = [gate | up] is written
// too when the caller passes x_out (the backward's input). Rows at or past
// the last end belong to no expert and are not written.
//
// Kernel shape (the launched configuration, Prod below):
//   * A block computes a 256-token x 128-column tile of gate and the same
//     tile of up (so each output's gate and up sit in the same lane), with
//     eight wavefronts (4 x 2) of 64 x 64 each: 2 x 2 v_mfma_f32_32x32x16_bf16
//     tiles for gate and 2 x 2 for up, 128 fp32 accumulators per lane, two
//     wavefronts per SIMD.
//   * K advances 64 at a time through double-buffered LDS tiles of A, W_gate
//     and W_up (rows padded by 16 bytes, which makes the 16-byte fragment
//     reads conflict-free; 144 KiB in all, one block per CU); the next K
//     step's global loads are in flight while the current one's MFMAs run.
//     One barrier per K step. Of 14 tile shapes measured at 131072 x 7168 x
//     2048 (64-256 tokens, 64-256 columns, K steps of 32 and 64, 1-3 waves per
//     SIMD; every shape gives bit-identical results, since each output is
//     accumulated in the same order), this one ran fastest.
//   * Tiles never straddle experts: each block finds its expert and row range
//     from offs on the device (no host copy of offs), so a grid sized for
//     the worst case, ceil(tokens / 256) + experts row tiles, covers any split.
//   * XCD-aware order: consecutive block ids land on different XCDs, so the
//     block id is remapped to give each XCD a contiguous range of tiles, and
//     the column tiles that share one A tile run on the same XCD (and L2).
//   * Epilogue: accumulators are rounded to bf16, the SwiGLU is applied, and
//     each output tile is staged through LDS so that global stores are
//     16-byte, row-contiguous accesses.
#include "epi_common.h"
#include "swiglu_math.h"

namespace moe_epi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kXcds = 8;  // MI355X: 8 XCDs, work-groups dispatched round-robin over them

// Tile configuration: a block computes BM tokens x BN columns of gate and the
// same columns of up, with WM x WN wavefronts (each BM/WM x BN/WN of both),
// stepping BK along hidden; OCC wavefronts per SIMD is the occupancy the
// compiler must leave room for (it caps the registers per lane at 512 / OCC).
template <int BM_, int BN_, int BK_, int WM_, int WN_, int OCC_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, OCC = OCC_;
    static constexpr int kThreads = 64 * WM * WN;
    static constexpr int MI = BM / (32 * WM);        // 32 x 32 MFMA tiles per wavefront, along tokens
    static constexpr int NI = BN / (32 * WN);        // ... along columns (for gate, and again for up)
    static constexpr int kLdk = BK + 8;              // LDS row stride of a K tile, in bf16 (16 bytes of padding)
    static constexpr int kAElems = BM * kLdk;
    static constexpr int kWElems = BN * kLdk;
    static constexpr int kStageElems = kAElems + 2 * kWElems;
    static constexpr int kLdo = BN + 8;              // LDS row stride of a staged output tile, in bf16
    static constexpr int kAChunks = BM * BK / 8 / kThreads;  // 16-byte chunks per thread per K step
    static constexpr int kWChunks = BN * BK / 8 / kThreads;
    static_assert(MI >= 1 && NI >= 1 && BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "whole MFMA tiles");
    static_assert(BK % 16 == 0 && kAChunks >= 1 && kWChunks >= 1 && BM * BK % (8 * kThreads) == 0 &&
                  BN * BK % (8 * kThreads) == 0, "whole 16-byte chunks per thread");
    // LDS holds two K-step buffers, then (after the K loop) one staged output tile
    static constexpr int kLdsElems = 2 * kStageElems > BM * kLdo ? 2 * kStageElems : BM * kLdo;
    static_assert(BM * BN % (8 * kThreads) == 0, "whole output chunks per thread");
};

// The configuration the library launches (see the shape notes above).
using Prod = Cfg<256, 128, 64, 4, 2, 2>;

struct TileRows {
    int64_t row0;   // first token of the tile
    int rows;       // valid tokens in the tile (0: no tile)
    int64_t expert;
};

// The mt-th row tile over all experts in order, each expert split into tiles
// of bm rows (the last one partial). Uniform across the block.
__device__ TileRows find_row_tile(const int32_t* __restrict__ offs, int64_t tokens, int64_t experts, int64_t mt,
                                  int bm) {
    int64_t start = 0, before = 0;
    for (int64_t e = 0; e < experts; ++e) {
        int64_t end = offs[e];
        end = end < start ? start : (end > tokens ? tokens : end);
        const int64_t n = (end - start + bm - 1) / bm;
        if (mt < before + n) {
            const int64_t row0 = start + (mt - before) * bm;
            const int64_t left = end - row0;
            return TileRows{row0, static_cast<int>(left < bm ? left : bm), e};
        }
        before += n;
        start = end;
    }
    return TileRows{0, 0, 0};
}

// Global -> registers: this thread's 16-byte chunks of an operand tile of
// `rows_tile` rows (rows [0, nrows) valid; columns k0 + [0, BK) of a
// row-major matrix with `ld` elements per row, those at or past kend zero).
template <class C, int N>
__device__ __forceinline__ void load_chunks(u32x4 (&r)[N], const uint16_t* __restrict__ base, int64_t ld, int nrows,
                                            int64_t k0, int64_t kend) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int c = static_cast<int>(threadIdx.x) + i * C::kThreads;
        const int row = c / (C::BK / 8), kq = c % (C::BK / 8);
        const int64_t k = k0 + kq * 8;
        if (row < nrows && k < kend)
            r[i] = *reinterpret_cast<const u32x4*>(base + row * ld + k);
        else
            r[i] = u32x4{0u, 0u, 0u, 0u};
    }
}

template <class C, int N>
__device__ __forceinline__ void store_chunks(uint16_t* tile, const u32x4 (&r)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int c = static_cast<int>(threadIdx.x) + i * C::kThreads;
        const int row = c / (C::BK / 8), kq = c % (C::BK / 8);
        *reinterpret_cast<u32x4*>(tile + row * C::kLdk + kq * 8) = r[i];
    }
}

template <class C>
__device__ __forceinline__ bf16x8 frag(const uint16_t* tile, int row, int k) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(tile + row * C::kLdk + k));
}

__device__ __forceinline__ float round_bf16(float v) { return __uint_as_float(static_cast<uint32_t>(to_bf16(v)) << 16); }

// Position in the block tile of accumulator element j of MFMA tile (mi, ni)
// held by lane l: v_mfma_f32_32x32x16 leaves C[8*(j/4) + 4*(l/32) + j%4][l%32]
// in register j (checked on the GPU).
template <class C>
__device__ __forceinline__ int acc_row(int wm, int mi, int j, int lane) {
    return wm * (C::BM / C::WM) + mi * 32 + 8 * (j / 4) + 4 * (lane / 32) + (j % 4);
}
template <class C>
__device__ __forceinline__ int acc_col(int wn, int ni, int lane) {
    return wn * (C::BN / C::WN) + ni * 32 + lane % 32;
}

// Write the staged [BM][kLdo] tile's valid rows and columns to a row-major
// bf16 matrix (ld elements per row) at (row0, col0) with 16-byte stores.
template <class C>
__device__ __forceinline__ void store_tile(const uint16_t* stage, uint16_t* __restrict__ out, int64_t ld,
                                           int64_t row0, int rows, int64_t col0, int64_t cend) {
    constexpr int kOutChunks = C::BM * C::BN / 8 / C::kThreads;
#pragma unroll
    for (int i = 0; i < kOutChunks; ++i) {
        const int c = static_cast<int>(threadIdx.x) + i * C::kThreads;
        const int row = c / (C::BN / 8), cq = c % (C::BN / 8);
        const int64_t col = col0 + cq * 8;
        if (row < rows && col < cend)
            *reinterpret_cast<u32x4*>(out + (row0 + row) * ld + col) =
                *reinterpret_cast<const u32x4*>(stage + row * C::kLdo + cq * 8);
    }
}

template <class C, bool kWriteX>
__global__ __launch_bounds__(C::kThreads) __attribute__((amdgpu_waves_per_eu(C::OCC))) void grouped_gate_up_swiglu_kernel(
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ w_gate, const uint16_t* __restrict__ w_up,
    const int32_t* __restrict__ offs, const float* __restrict__ probs, uint16_t* __restrict__ y,
    uint16_t* __restrict__ x_out, int64_t tokens, int64_t hidden, int64_t inter, int64_t experts, float L,
    int64_t n_tiles, int64_t n_blocks) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[C::kLdsElems];
    constexpr int MI = C::MI, NI = C::NI;

    // XCD-aware order: block b runs on XCD b % 8; XCD x takes logical tiles
    // [x * per, (x + 1) * per). The grid is 8 * per blocks.
    const int64_t per = static_cast<int64_t>(gridDim.x) / kXcds;
    const int64_t logical = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
    if (logical >= n_blocks) return;
    const int64_t mt = logical / n_tiles;
    const int64_t col0 = (logical % n_tiles) * C::BN;
    const TileRows tr = find_row_tile(offs, tokens, experts, mt, C::BM);
    if (tr.rows == 0) return;
    const int ncols = static_cast<int>(inter - col0 < C::BN ? inter - col0 : C::BN);

    const uint16_t* a_tile = a + tr.row0 * hidden;
    const uint16_t* g_tile = w_gate + (tr.expert * inter + col0) * hidden;
    const uint16_t* u_tile = w_up + (tr.expert * inter + col0) * hidden;

    const int lane = static_cast<int>(threadIdx.x) % 64;
    const int wave = static_cast<int>(threadIdx.x) / 64;
    const int wm = wave / C::WN, wn = wave % C::WN;

    f32x16 acc_g[MI][NI], acc_u[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
            acc_g[mi][ni] = f32x16{};
            acc_u[mi][ni] = f32x16{};
        }

    u32x4 ra[C::kAChunks], rg[C::kWChunks], ru[C::kWChunks];
    const int64_t nk = (hidden + C::BK - 1) / C::BK;
    load_chunks<C>(ra, a_tile, hidden, tr.rows, 0, hidden);
    load_chunks<C>(rg, g_tile, hidden, ncols, 0, hidden);
    load_chunks<C>(ru, u_tile, hidden, ncols, 0, hidden);
    store_chunks<C>(lds, ra);
    store_chunks<C>(lds + C::kAElems, rg);
    store_chunks<C>(lds + C::kAElems + C::kWElems, ru);
    __syncthreads();

    for (int64_t kt = 0; kt < nk; ++kt) {
        uint16_t* cur = lds + (kt & 1) * C::kStageElems;
        const bool more = kt + 1 < nk;
        if (more) {
            const int64_t k0 = (kt + 1) * C::BK;
            load_chunks<C>(ra, a_tile, hidden, tr.rows, k0, hidden);
            load_chunks<C>(rg, g_tile, hidden, ncols, k0, hidden);
            load_chunks<C>(ru, u_tile, hidden, ncols, k0, hidden);
        }
        const uint16_t* sa = cur;
        const uint16_t* sg = cur + C::kAElems;
        const uint16_t* su = cur + C::kAElems + C::kWElems;
#pragma unroll
        for (int kk = 0; kk < C::BK / 16; ++kk) {
            const int k = kk * 16 + (lane / 32) * 8;
            bf16x8 fa[MI], fg[NI], fu[NI];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) fa[mi] = frag<C>(sa, wm * (C::BM / C::WM) + mi * 32 + lane % 32, k);
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                fg[ni] = frag<C>(sg, wn * (C::BN / C::WN) + ni * 32 + lane % 32, k);
                fu[ni] = frag<C>(su, wn * (C::BN / C::WN) + ni * 32 + lane % 32, k);
            }
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) {
                    acc_g[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fg[ni], acc_g[mi][ni], 0, 0, 0);
                    acc_u[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fu[ni], acc_u[mi][ni], 0, 0, 0);
                }
        }
        if (more) {
            uint16_t* nxt = lds + ((kt + 1) & 1) * C::kStageElems;
            store_chunks<C>(nxt, ra);
            store_chunks<C>(nxt + C::kAElems, rg);
            store_chunks<C>(nxt + C::kAElems + C::kWElems, ru);
        }
        __syncthreads();
    }

    // ---- epilogue: y (and x) through an LDS staging tile -------------------
    uint16_t* stage = lds;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int r = acc_row<C>(wm, mi, j, lane);
            const float p = r < tr.rows ? probs[tr.row0 + r] : 0.0f;
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const float g = round_bf16(acc_g[mi][ni][j]);
                const float u = round_bf16(acc_u[mi][ni][j]);
                stage[r * C::kLdo + acc_col<C>(wn, ni, lane)] = to_bf16(fwd_elem(g, u, p, L));
            }
        }
    __syncthreads();
    store_tile<C>(stage, y, inter, tr.row0, tr.rows, col0, inter);
    if constexpr (kWriteX) {
        __syncthreads();
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    stage[acc_row<C>(wm, mi, j, lane) * C::kLdo + acc_col<C>(wn, ni, lane)] =
                        to_bf16(acc_g[mi][ni][j]);
        __syncthreads();
        store_tile<C>(stage, x_out, 2 * inter, tr.row0, tr.rows, col0, inter);
        __syncthreads();
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    stage[acc_row<C>(wm, mi, j, lane) * C::kLdo + acc_col<C>(wn, ni, lane)] =
                        to_bf16(acc_u[mi][ni][j]);
        __syncthreads();
        store_tile<C>(stage, x_out + inter, 2 * inter, tr.row0, tr.rows, col0, inter);
    }
}

// Grid: row tiles (worst case ceil(tokens / BM) + experts) times column
// tiles, rounded up to a multiple of the XCD count. Returns 0 when it does not
// fit a 1-D grid.
template <class C>
int64_t grouped_grid(int64_t tokens, int64_t inter, int64_t experts, int64_t* n_tiles, int64_t* n_blocks) {
    *n_tiles = (inter + C::BN - 1) / C::BN;
    const int64_t m_bound = (tokens + C::BM - 1) / C::BM + experts;
    *n_blocks = m_bound * *n_tiles;
    const int64_t grid = (*n_blocks + kXcds - 1) / kXcds * kXcds;
    return grid < (static_cast<int64_t>(1) << 31) ? grid : 0;
}

template <class C>
int launch_grouped(const uint16_t* a, const uint16_t* w_gate, const uint16_t* w_up, const int32_t* offs,
                   const float* probs, uint16_t* y, uint16_t* x_out, int64_t tokens, int64_t hidden, int64_t inter,
                   int64_t experts, float limit, hipStream_t st) {
    int64_t n_tiles, n_blocks;
    const int64_t grid = grouped_grid<C>(tokens, inter, experts, &n_tiles, &n_blocks);
    if (grid == 0) return MOE_EPI_ERR_BAD_SHAPE;
    (void)hipGetLastError();
    if (x_out)
        hipLaunchKernelGGL((grouped_gate_up_swiglu_kernel<C, true>), dim3(static_cast<unsigned>(grid)),
                           dim3(C::kThreads), 0, st, a, w_gate, w_up, offs, probs, y, x_out, tokens, hidden, inter,
                           experts, limit, n_tiles, n_blocks);
    else
        hipLaunchKernelGGL((grouped_gate_up_swiglu_kernel<C, false>), dim3(static_cast<unsigned>(grid)),
                           dim3(C::kThreads), 0, st, a, w_gate, w_up, offs, probs, y, x_out, tokens, hidden, inter,
                           experts, limit, n_tiles, n_blocks);
    return launch_status();
}

}  // namespace
}  // namespace moe_epi

using namespace moe_epi;

extern "C" int grouped_gate_up_swiglu_fwd(const uint16_t* a, const uint16_t* w_gate, const uint16_t* w_up,
                                          const int32_t* offs, const float* probs, uint16_t* y, uint16_t* x_out,
                                          int64_t tokens, int64_t hidden, int64_t inter, int64_t experts,
                                          float limit, void* stream) {
    if (tokens < 0 || tokens > INT32_MAX || hidden <= 0 || inter <= 0 || experts <= 0 || hidden % 8 != 0 ||
        inter % 8 != 0)
        return MOE_EPI_ERR_BAD_SHAPE;
    int64_t ab, wb, yb, xb, pb, ob;
    if (experts > INT64_MAX / 4 / inter)  // before experts * inter is formed
        return MOE_EPI_ERR_BAD_SHAPE;
    if (!bytes_ok(tokens, hidden, 2, &ab) || !bytes_ok(experts * inter, hidden, 2, &wb) ||
        !bytes_ok(tokens, inter, 2, &yb) || !bytes_ok(tokens, 2 * inter, 2, &xb) || !bytes_ok(tokens, 1, 4, &pb) ||
        !bytes_ok(experts, 1, 4, &ob))
        return MOE_EPI_ERR_BAD_SHAPE;
    if (!(limit > 0.0f) || !isfinite(limit)) return MOE_EPI_ERR_BAD_LIMIT;
    if (tokens == 0) return MOE_EPI_SUCCESS;
    if (!a || !w_gate || !w_up || !offs || !probs || !y) return MOE_EPI_ERR_NULL_POINTER;
    if (!aligned(a, 16) || !aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(y, 16) ||
        (x_out && !aligned(x_out, 16)) || !aligned(offs, 4) || !aligned(probs, 4))
        return MOE_EPI_ERR_MISALIGNED;
    const Range ra = range_of(a, ab), rg = range_of(w_gate, wb), ru = range_of(w_up, wb), ro = range_of(offs, ob),
                rp = range_of(probs, pb), ry = range_of(y, yb), rx = range_of(x_out, x_out ? xb : 0);
    for (const Range& out : {ry, rx})
        if (overlaps(out, ra) || overlaps(out, rg) || overlaps(out, ru) || overlaps(out, ro) || overlaps(out, rp))
            return MOE_EPI_ERR_ALIAS;
    if (overlaps(ry, rx)) return MOE_EPI_ERR_ALIAS;
    return launch_grouped<Prod>(a, w_gate, w_up, offs, probs, y, x_out, tokens, hidden, inter, experts, limit,
                                as_stream(stream));
}
