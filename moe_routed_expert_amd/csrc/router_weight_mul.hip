// fp32 router-weight multiply: forward and backward for gfx950.
//
// Operation (page "nemo_automodel.components.moe.optimized_ops", entries
// _RouterWeightMulFunction, _rw_fwd_core, _rw_bwd_x_core, _rw_bwd_probs_core):
// on the expert down-projection output x [tokens, hidden] with one fp32
// routing probability per row,
//   out        = round_out(fp32(x) * p)             (bitwise equal to the eager multiply)
//   grad_x     = round_x(fp32(grad_out) * p)
//   grad_probs = sum_k fp32(grad_out) * fp32(x)     (fp32)
// where the output (and so grad_out) is x's dtype or fp32. The page computes
// the two gradients with two cores, i.e. two passes over grad_out; here both
// come out of one pass (grad_out and x read once).
//
// Kernel shape: as for the SwiGLU kernels, a group of G lanes owns a row and
// walks it in nontemporal vectors of 8 elements, V vectors per lane in
// flight, spread over several wavefronts per row (see the launchers); the row
// sum is a register accumulator reduced with cross-lane shuffles and, across
// wavefronts, a few LDS slots. The forward needs no reduction but uses the
// same row walk, which loads the row's probability once and needs no division
// to find a vector's row.
#include "epi_common.h"

namespace moe_epi {
namespace {

// block size of the per-element kernels
constexpr int kBlock = 256;

// G lanes own a row (G <= 64: part of a wavefront; G = 64*W: W wavefronts),
// B threads per block. The row loop advances whole blocks so that every thread
// of a block runs the same iterations (row_sum may hold a barrier). TX is the
// dtype of x and grad_x, TO that of out and grad_out.
// kAlign: the block's wavefronts meet at a barrier before any of them issues
// its row loads (align_block_loads, epi_common.h).
template <int TX, int TO, int G, int V, int B, bool kAlign>
__global__ __launch_bounds__(B) void router_weight_mul_fwd_kernel(const void* __restrict__ x,
                                                                  const float* __restrict__ probs,
                                                                  void* __restrict__ out, int64_t rows,
                                                                  int64_t hidden) {
    using EX = Elem<TX>;
    using EO = Elem<TO>;
    constexpr bool kSplit = TX == MOE_EPI_F32 || TO == MOE_EPI_F32;  // the vector map (epi_common.h)
    constexpr int kRows = B / G;
    const uint32_t lane = threadIdx.x % G;
    const uint32_t nvec = static_cast<uint32_t>(hidden / 8);
    for (int64_t rb = static_cast<int64_t>(blockIdx.x) * kRows; rb < rows;
         rb += static_cast<int64_t>(gridDim.x) * kRows) {
        const int64_t r = rb + group_in_block<G>();
        const float p = r < rows ? probs[r] : 0.0f;
        if constexpr (kAlign) align_block_loads();
        if (r >= rows) continue;
        const void* xr = row_at<TX>(x, r * hidden);
        void* outr = row_at<TO>(out, r * hidden);
        for (uint32_t c0 = lane; c0 < nvec; c0 += G * V) {
            typename EX::Raw v[V];
            Quads q[V];
#pragma unroll
            for (int k = 0; k < V; ++k) q[k] = quads_of<G, kSplit>(c0 + k * G, lane, nvec);
#pragma unroll
            for (int k = 0; k < V; ++k)
                if (c0 + k * G < nvec) v[k] = EX::template load<kSplit>(xr, q[k]);
#pragma unroll
            for (int k = 0; k < V; ++k) {
                if (c0 + k * G < nvec) {
                    float f[8];
                    EX::unpack(v[k], f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) f[e] = f[e] * p;
                    EO::template store<kSplit>(outr, q[k], EO::pack(f));
                }
            }
        }
    }
}

template <int TX, int TO, int G, int V, int B, bool kGradProbs, bool kAlign>
__global__ __launch_bounds__(B) __attribute__((amdgpu_waves_per_eu(waves_for_two_blocks(B)))) void
router_weight_mul_bwd_kernel(const void* __restrict__ grad_out, const void* __restrict__ x,
                             const float* __restrict__ probs, void* __restrict__ grad_x,
                             float* __restrict__ grad_probs, int64_t rows, int64_t hidden) {
    using EX = Elem<TX>;
    using EO = Elem<TO>;
    constexpr bool kSplit = TX == MOE_EPI_F32 || TO == MOE_EPI_F32;  // the vector map (epi_common.h)
    constexpr int kRows = B / G;
    __shared__ float part[B / 64 > 0 ? B / 64 : 1];
    const uint32_t lane = threadIdx.x % G;
    const uint32_t nvec = static_cast<uint32_t>(hidden / 8);
    for (int64_t rb = static_cast<int64_t>(blockIdx.x) * kRows; rb < rows;
         rb += static_cast<int64_t>(gridDim.x) * kRows) {
        const int64_t r = rb + group_in_block<G>();
        float acc = 0.0f;
        const float p = r < rows ? probs[r] : 0.0f;
        if constexpr (kAlign) align_block_loads();
        if (r < rows) {
            const void* gor = row_at<TO>(grad_out, r * hidden);
            const void* xr = kGradProbs ? row_at<TX>(x, r * hidden) : nullptr;
            void* gxr = row_at<TX>(grad_x, r * hidden);
            for (uint32_t c0 = lane; c0 < nvec; c0 += G * V) {
                typename EO::Raw g[V];
                typename EX::Raw xv[V];
                Quads q[V];
#pragma unroll
                for (int k = 0; k < V; ++k) q[k] = quads_of<G, kSplit>(c0 + k * G, lane, nvec);
#pragma unroll
                for (int k = 0; k < V; ++k)
                    if (c0 + k * G < nvec) g[k] = EO::template load<kSplit>(gor, q[k]);
                if (kGradProbs) {
#pragma unroll
                    for (int k = 0; k < V; ++k)
                        if (c0 + k * G < nvec) xv[k] = EX::template load<kSplit>(xr, q[k]);
                }
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    if (c0 + k * G < nvec) {
                        float gf[8], o[8];
                        EO::unpack(g[k], gf);
#pragma unroll
                        for (int e = 0; e < 8; ++e) o[e] = gf[e] * p;
                        if (kGradProbs) {
                            float xf[8];
                            EX::unpack(xv[k], xf);
                            // bf16 x bf16 products are exact in fp32; for wider
                            // types the fused multiply-add rounds once
#pragma unroll
                            for (int e = 0; e < 8; ++e) acc = __fmaf_rn(gf[e], xf[e], acc);
                        }
                        EX::template store<kSplit>(gxr, q[k], EX::pack(o));
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

// per-element kernels (any hidden, element-aligned tensors)
template <int TX, int TO>
__global__ __launch_bounds__(kBlock) void router_weight_mul_fwd_scalar_kernel(const void* __restrict__ x,
                                                                             const float* __restrict__ probs,
                                                                             void* __restrict__ out, int64_t rows,
                                                                             int64_t hidden) {
    constexpr int kRows = kBlock / 64;
    const int lane = threadIdx.x % 64;
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * kRows + threadIdx.x / 64; r < rows;
         r += static_cast<int64_t>(gridDim.x) * kRows) {
        const float p = probs[r];
        for (int64_t k = lane; k < hidden; k += 64)
            Elem<TO>::store1(out, r * hidden + k, Elem<TX>::load1(x, r * hidden + k) * p);
    }
}

template <int TX, int TO, bool kGradProbs>
__global__ __launch_bounds__(kBlock) void router_weight_mul_bwd_scalar_kernel(
    const void* __restrict__ grad_out, const void* __restrict__ x, const float* __restrict__ probs,
    void* __restrict__ grad_x, float* __restrict__ grad_probs, int64_t rows, int64_t hidden) {
    constexpr int kRows = kBlock / 64;
    const int lane = threadIdx.x % 64;
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * kRows + threadIdx.x / 64; r < rows;
         r += static_cast<int64_t>(gridDim.x) * kRows) {
        const float p = probs[r];
        float acc = 0.0f;
        for (int64_t k = lane; k < hidden; k += 64) {
            const float g = Elem<TO>::load1(grad_out, r * hidden + k);
            Elem<TX>::store1(grad_x, r * hidden + k, g * p);
            if (kGradProbs) acc = __fmaf_rn(g, Elem<TX>::load1(x, r * hidden + k), acc);
        }
        if (kGradProbs) {
            acc = group_sum<64>(acc);
            if (lane == 0) grad_probs[r] = acc;
        }
    }
}

// Launch shapes: G lanes per row, V vectors per lane per pass, B threads per
// block (B / G rows per block). For rows of 192 to 1024 vectors (1536 to 8192
// columns) they come from a sweep on MI355X of 59 forward and 40 backward
// shapes per dtype pair at 2048, 4096 and 7168 columns (131072, 65536 and
// 65536 rows), one table per class of pair (16-bit x and output; 16-bit x
// with float32 output; float32 both): each entry is the shape whose worst
// case over the pairs sharing it was best, every entry within 2.5% of that
// case's fastest shape (the shapes they replace lost up to 15%). As for the
// SwiGLU kernels, one row per block and few rows in flight per CU, each
// streamed by many wavefronts, did best. Narrower rows keep the earlier rules
// (a wavefront or less per row under 64 vectors, then 1-2 wavefronts), and so
// do wider ones (the forward with 2 wavefronts per row and up to 16 vectors
// per lane, the backward with 2 vectors per lane and up to 16 wavefronts per
// row; longer rows take several passes).
enum class Cls { k16, kMixed, k32 };

template <int TX, int TO>
constexpr Cls cls_of() {
    return TX == MOE_EPI_F32 ? Cls::k32 : (TO == MOE_EPI_F32 ? Cls::kMixed : Cls::k16);
}

template <int TX, int TO, int G, int V, int B, bool kAlign = false>
void launch_fwd(const void* x, const float* probs, void* out, int64_t rows, int64_t hidden, hipStream_t st) {
    hipLaunchKernelGGL((router_weight_mul_fwd_kernel<TX, TO, G, V, B, kAlign>), dim3(grid_for_rows(rows, B / G)),
                       dim3(B), 0, st, x, probs, out, rows, hidden);
}

template <int TX, int TO, int G, int V, int B, bool kAlign = false>
void launch_bwd(const void* go, const void* x, const float* probs, void* gx, float* gp, int64_t rows, int64_t hidden,
                hipStream_t st) {
    const dim3 grid(grid_for_rows(rows, B / G));
    if (gp)
        hipLaunchKernelGGL((router_weight_mul_bwd_kernel<TX, TO, G, V, B, true, kAlign>), grid, dim3(B), 0, st, go, x,
                           probs, gx, gp, rows, hidden);
    else
        hipLaunchKernelGGL((router_weight_mul_bwd_kernel<TX, TO, G, V, B, false, kAlign>), grid, dim3(B), 0, st, go, x,
                           probs, gx, gp, rows, hidden);
}

template <int TX, int TO>
void dispatch_fwd(const void* x, const float* probs, void* out, int64_t rows, int64_t hidden, hipStream_t st) {
    const int64_t nvec = hidden / 8;
    if (nvec < 64) {
        switch (small_group(nvec)) {
            case 8: return launch_fwd<TX, TO, 8, 1, 256>(x, probs, out, rows, hidden, st);
            case 16: return launch_fwd<TX, TO, 16, 1, 256>(x, probs, out, rows, hidden, st);
            default: return launch_fwd<TX, TO, 32, 1, 256>(x, probs, out, rows, hidden, st);
        }
    }
    if (nvec < 128) return launch_fwd<TX, TO, 64, 2, 256>(x, probs, out, rows, hidden, st);
    if (nvec == 128) return launch_fwd<TX, TO, 128, 1, 256>(x, probs, out, rows, hidden, st);
    if (nvec < 192) return launch_fwd<TX, TO, 128, 2, 256>(x, probs, out, rows, hidden, st);
    // 896 vectors (hidden 7168, the pages' model width) with 16-bit x: shapes
    // from a second sweep, per dtype pair, with the option of aligned row loads
    // (align_block_loads, epi_common.h); caches flushed before every launch
    if constexpr (TX == MOE_EPI_BF16 || TX == MOE_EPI_F16) {
        if (nvec == 896) {
            // bf16 out: 320 lanes of two vectors a pass, three rows per block,
            // aligned: 79.7% of HBM peak against 76.3% for one unaligned row
            // per block (two rows per block: the same); fp16 out: two rows per
            // block, aligned: 80.7-81.8% against 77.4-77.6% for one unaligned
            // row (three rows: 79.7-80.3%); fp32 out: 896 lanes, aligned: 83.2%
            // (bf16 x) and 83.0% (fp16 x) against 74.8% and 73.7% for 512
            // lanes unaligned
            if constexpr (TX == MOE_EPI_BF16 && TO == MOE_EPI_BF16)
                return launch_fwd<TX, TO, 320, 2, 960, true>(x, probs, out, rows, hidden, st);
            if constexpr (TX == MOE_EPI_F16 && TO == MOE_EPI_F16)
                return launch_fwd<TX, TO, 320, 2, 640, true>(x, probs, out, rows, hidden, st);
            if constexpr (TO == MOE_EPI_F32) return launch_fwd<TX, TO, 896, 1, 896, true>(x, probs, out, rows, hidden, st);
        }
    }
    if constexpr (TX == MOE_EPI_F32) {
        // fp32 x and out, 896 vectors: two vectors per lane of 896, aligned:
        // 79.8% of HBM peak against 73.4% for two 512-lane passes unaligned
        if (nvec == 896) return launch_fwd<TX, TO, 896, 2, 896, true>(x, probs, out, rows, hidden, st);
    }
    if (nvec <= 1024) {
        constexpr Cls c = cls_of<TX, TO>();
        if constexpr (c == Cls::k16) {
            if (nvec <= 256) return launch_fwd<TX, TO, 192, 1, 192>(x, probs, out, rows, hidden, st);
            if (nvec <= 512) return launch_fwd<TX, TO, 192, 2, 384>(x, probs, out, rows, hidden, st);
            return launch_fwd<TX, TO, 320, 2, 320>(x, probs, out, rows, hidden, st);
        } else if constexpr (c == Cls::kMixed) {
            if (nvec <= 256) return launch_fwd<TX, TO, 640, 1, 640>(x, probs, out, rows, hidden, st);
            if (nvec <= 512) return launch_fwd<TX, TO, 896, 2, 896>(x, probs, out, rows, hidden, st);
            return launch_fwd<TX, TO, 512, 1, 512>(x, probs, out, rows, hidden, st);
        } else {
            if (nvec <= 256) return launch_fwd<TX, TO, 1024, 1, 1024>(x, probs, out, rows, hidden, st);
            if (nvec <= 512) return launch_fwd<TX, TO, 384, 1, 384>(x, probs, out, rows, hidden, st);
            return launch_fwd<TX, TO, 512, 1, 1024>(x, probs, out, rows, hidden, st);
        }
    }
    if (nvec <= 12 * 128) return launch_fwd<TX, TO, 128, 12, 256>(x, probs, out, rows, hidden, st);
    return launch_fwd<TX, TO, 128, 16, 256>(x, probs, out, rows, hidden, st);  // wider rows: passes
}

template <int TX, int TO>
void dispatch_bwd(const void* go, const void* x, const float* probs, void* gx, float* gp, int64_t rows,
                  int64_t hidden, hipStream_t st) {
    const int64_t nvec = hidden / 8;
    if (nvec < 64) {
        switch (small_group(nvec)) {
            case 8: return launch_bwd<TX, TO, 8, 1, 256>(go, x, probs, gx, gp, rows, hidden, st);
            case 16: return launch_bwd<TX, TO, 16, 1, 256>(go, x, probs, gx, gp, rows, hidden, st);
            default: return launch_bwd<TX, TO, 32, 1, 256>(go, x, probs, gx, gp, rows, hidden, st);
        }
    }
    if (nvec <= 128) return launch_bwd<TX, TO, 64, 2, 128>(go, x, probs, gx, gp, rows, hidden, st);
    if (nvec < 192) return launch_bwd<TX, TO, 128, 2, 256>(go, x, probs, gx, gp, rows, hidden, st);
    // 896 vectors (hidden 7168): as for the forward, a second sweep per pair
    if constexpr (TX == MOE_EPI_BF16 || TX == MOE_EPI_F16) {
        if (nvec == 896) {
            // fp32 grad_out: 896 lanes, aligned: 83.8% of HBM peak against 81.1%
            // unaligned (bf16 x), 83.8% against 80.9% (fp16 x)
            if constexpr (TO == MOE_EPI_F32)
                return launch_bwd<TX, TO, 896, 1, 896, true>(go, x, probs, gx, gp, rows, hidden, st);
            if constexpr (TO == TX) {
                // without the probability gradient the backward only streams
                // grad_out into grad_x, a 1:1 copy: the forward's 320 lanes of two
                // vectors, two rows per block, aligned: 80.3% against 74.3% (bf16)
                // and 73.9% (fp16) for the shape below
                if (!gp) return launch_bwd<TX, TO, 320, 2, 640, true>(go, x, probs, gx, gp, rows, hidden, st);
                // bf16 grad_out, aligned: 81.3% against 77.7% unaligned; fp16 keeps
                // the unaligned 16-bit shape below (82.0-82.5%, aligned 81.8%)
                if constexpr (TX == MOE_EPI_BF16)
                    return launch_bwd<TX, TO, 448, 2, 896, true>(go, x, probs, gx, gp, rows, hidden, st);
            }
        }
    }
    if constexpr (TX == MOE_EPI_F32) {
        // fp32: two vectors per lane of 896, aligned: 80.3% against 76.6%
        if (nvec == 896) return launch_bwd<TX, TO, 896, 2, 896, true>(go, x, probs, gx, gp, rows, hidden, st);
    }
    if (nvec <= 1024) {
        constexpr Cls c = cls_of<TX, TO>();
        if constexpr (c == Cls::k16) {
            if (nvec <= 256) return launch_bwd<TX, TO, 256, 2, 512>(go, x, probs, gx, gp, rows, hidden, st);
            if (nvec <= 512) return launch_bwd<TX, TO, 512, 2, 1024>(go, x, probs, gx, gp, rows, hidden, st);
            return launch_bwd<TX, TO, 448, 2, 896>(go, x, probs, gx, gp, rows, hidden, st);
        } else if constexpr (c == Cls::kMixed) {
            if (nvec <= 256) return launch_bwd<TX, TO, 320, 1, 640>(go, x, probs, gx, gp, rows, hidden, st);
            if (nvec <= 512) return launch_bwd<TX, TO, 512, 2, 1024>(go, x, probs, gx, gp, rows, hidden, st);
            return launch_bwd<TX, TO, 896, 1, 896>(go, x, probs, gx, gp, rows, hidden, st);
        } else {
            if (nvec <= 256) return launch_bwd<TX, TO, 512, 1, 1024>(go, x, probs, gx, gp, rows, hidden, st);
            if (nvec <= 512) return launch_bwd<TX, TO, 896, 1, 896>(go, x, probs, gx, gp, rows, hidden, st);
            return launch_bwd<TX, TO, 896, 2, 896>(go, x, probs, gx, gp, rows, hidden, st);
        }
    }
    if (nvec <= 12 * 128) return launch_bwd<TX, TO, 768, 2, 768>(go, x, probs, gx, gp, rows, hidden, st);
    return launch_bwd<TX, TO, 1024, 2, 1024>(go, x, probs, gx, gp, rows, hidden, st);  // wider rows: passes
}

// The (x, output) dtype pairs: the output is x's dtype or float32.
enum class Pair { kBB, kBF, kHH, kHF, kFF, kBad };

Pair pair_of(int x_dtype, int out_dtype) {
    if (x_dtype == MOE_EPI_BF16 && out_dtype == MOE_EPI_BF16) return Pair::kBB;
    if (x_dtype == MOE_EPI_BF16 && out_dtype == MOE_EPI_F32) return Pair::kBF;
    if (x_dtype == MOE_EPI_F16 && out_dtype == MOE_EPI_F16) return Pair::kHH;
    if (x_dtype == MOE_EPI_F16 && out_dtype == MOE_EPI_F32) return Pair::kHF;
    if (x_dtype == MOE_EPI_F32 && out_dtype == MOE_EPI_F32) return Pair::kFF;
    return Pair::kBad;
}

template <int TX, int TO>
void run_fwd(const void* x, const float* probs, void* out, int64_t rows, int64_t hidden, bool vec, hipStream_t st) {
    if (vec)
        dispatch_fwd<TX, TO>(x, probs, out, rows, hidden, st);
    else
        hipLaunchKernelGGL((router_weight_mul_fwd_scalar_kernel<TX, TO>), dim3(grid_for_rows(rows, kBlock / 64)),
                           dim3(kBlock), 0, st, x, probs, out, rows, hidden);
}

template <int TX, int TO>
void run_bwd(const void* go, const void* x, const float* probs, void* gx, float* gp, int64_t rows, int64_t hidden,
             bool vec, hipStream_t st) {
    if (vec) {
        dispatch_bwd<TX, TO>(go, x, probs, gx, gp, rows, hidden, st);
        return;
    }
    const dim3 grid(grid_for_rows(rows, kBlock / 64));
    if (gp)
        hipLaunchKernelGGL((router_weight_mul_bwd_scalar_kernel<TX, TO, true>), grid, dim3(kBlock), 0, st, go, x,
                           probs, gx, gp, rows, hidden);
    else
        hipLaunchKernelGGL((router_weight_mul_bwd_scalar_kernel<TX, TO, false>), grid, dim3(kBlock), 0, st, go, x,
                           probs, gx, gp, rows, hidden);
}

int check_router(int64_t rows, int64_t hidden, int x_dtype, int out_dtype, int64_t* x_bytes, int64_t* o_bytes,
                 int64_t* p_bytes) {
    if (!dtype_ok(x_dtype) || !dtype_ok(out_dtype) || pair_of(x_dtype, out_dtype) == Pair::kBad)
        return MOE_EPI_ERR_BAD_DTYPE;
    if (rows < 0 || hidden <= 0) return MOE_EPI_ERR_BAD_SHAPE;
    if (!bytes_ok(rows, hidden, elem_bytes(x_dtype), x_bytes) || !bytes_ok(rows, hidden, elem_bytes(out_dtype), o_bytes) ||
        !bytes_ok(rows, 1, 4, p_bytes))
        return MOE_EPI_ERR_BAD_SHAPE;
    return MOE_EPI_SUCCESS;
}

int router_fwd_impl(const void* x, int x_dtype, const float* probs, void* out, int out_dtype, int64_t rows,
                    int64_t hidden, void* stream) {
    int64_t xb, ob, pb;
    int st = check_router(rows, hidden, x_dtype, out_dtype, &xb, &ob, &pb);
    if (st != MOE_EPI_SUCCESS) return st;
    if (rows == 0) return MOE_EPI_SUCCESS;
    if (!x || !probs || !out) return MOE_EPI_ERR_NULL_POINTER;
    if (!aligned(x, elem_bytes(x_dtype)) || !aligned(out, elem_bytes(out_dtype)) || !aligned(probs, 4))
        return MOE_EPI_ERR_MISALIGNED;
    const Range rx = range_of(x, xb), rp = range_of(probs, pb), ro = range_of(out, ob);
    if (overlaps(ro, rx) || overlaps(ro, rp)) return MOE_EPI_ERR_ALIAS;

    hipStream_t s = as_stream(stream);
    (void)hipGetLastError();
    const int wide = elem_bytes(x_dtype) > elem_bytes(out_dtype) ? elem_bytes(x_dtype) : elem_bytes(out_dtype);
    const bool vec = hidden % 8 == 0 && row_fits_u32_offsets(hidden, wide) && aligned(x, 16) && aligned(out, 16);
    switch (pair_of(x_dtype, out_dtype)) {
        case Pair::kBB: run_fwd<MOE_EPI_BF16, MOE_EPI_BF16>(x, probs, out, rows, hidden, vec, s); break;
        case Pair::kBF: run_fwd<MOE_EPI_BF16, MOE_EPI_F32>(x, probs, out, rows, hidden, vec, s); break;
        case Pair::kHH: run_fwd<MOE_EPI_F16, MOE_EPI_F16>(x, probs, out, rows, hidden, vec, s); break;
        case Pair::kHF: run_fwd<MOE_EPI_F16, MOE_EPI_F32>(x, probs, out, rows, hidden, vec, s); break;
        default: run_fwd<MOE_EPI_F32, MOE_EPI_F32>(x, probs, out, rows, hidden, vec, s); break;
    }
    return launch_status();
}

int router_bwd_impl(const void* grad_out, int go_dtype, const void* x, int x_dtype, const float* probs, void* grad_x,
                    float* grad_probs, int64_t rows, int64_t hidden, void* stream) {
    int64_t xb, ob, pb;
    int st = check_router(rows, hidden, x_dtype, go_dtype, &xb, &ob, &pb);
    if (st != MOE_EPI_SUCCESS) return st;
    if (rows == 0) return MOE_EPI_SUCCESS;
    if (!grad_out || !probs || !grad_x || (grad_probs && !x)) return MOE_EPI_ERR_NULL_POINTER;
    if (!grad_probs) x = nullptr;  // x is only read for the probability gradient
    const int xe = elem_bytes(x_dtype);
    if (!aligned(grad_out, elem_bytes(go_dtype)) || !aligned(grad_x, xe) || !aligned(probs, 4) ||
        (x && !aligned(x, xe)) || (grad_probs && !aligned(grad_probs, 4)))
        return MOE_EPI_ERR_MISALIGNED;
    const Range rgo = range_of(grad_out, ob), rx = range_of(x, x ? xb : 0), rp = range_of(probs, pb);
    const Range rgx = range_of(grad_x, xb), rgp = range_of(grad_probs, grad_probs ? pb : 0);
    if (overlaps(rgx, rgo) || overlaps(rgx, rx) || overlaps(rgx, rp) || overlaps(rgp, rgo) || overlaps(rgp, rx) ||
        overlaps(rgp, rp) || overlaps(rgp, rgx))
        return MOE_EPI_ERR_ALIAS;

    hipStream_t s = as_stream(stream);
    (void)hipGetLastError();
    const int wide = xe > elem_bytes(go_dtype) ? xe : elem_bytes(go_dtype);
    const bool vec = hidden % 8 == 0 && row_fits_u32_offsets(hidden, wide) && aligned(grad_out, 16) &&
                     aligned(grad_x, 16) && (!x || aligned(x, 16));
    switch (pair_of(x_dtype, go_dtype)) {
        case Pair::kBB: run_bwd<MOE_EPI_BF16, MOE_EPI_BF16>(grad_out, x, probs, grad_x, grad_probs, rows, hidden, vec, s); break;
        case Pair::kBF: run_bwd<MOE_EPI_BF16, MOE_EPI_F32>(grad_out, x, probs, grad_x, grad_probs, rows, hidden, vec, s); break;
        case Pair::kHH: run_bwd<MOE_EPI_F16, MOE_EPI_F16>(grad_out, x, probs, grad_x, grad_probs, rows, hidden, vec, s); break;
        case Pair::kHF: run_bwd<MOE_EPI_F16, MOE_EPI_F32>(grad_out, x, probs, grad_x, grad_probs, rows, hidden, vec, s); break;
        default: run_bwd<MOE_EPI_F32, MOE_EPI_F32>(grad_out, x, probs, grad_x, grad_probs, rows, hidden, vec, s); break;
    }
    return launch_status();
}

}  // namespace
}  // namespace moe_epi

extern "C" int router_weight_mul_fwd(const uint16_t* x, const float* probs, uint16_t* out, int64_t rows,
                                     int64_t hidden, void* stream) {
    return moe_epi::router_fwd_impl(x, MOE_EPI_BF16, probs, out, MOE_EPI_BF16, rows, hidden, stream);
}

extern "C" int router_weight_mul_bwd(const uint16_t* grad_out, const uint16_t* x, const float* probs,
                                     uint16_t* grad_x, float* grad_probs, int64_t rows, int64_t hidden,
                                     void* stream) {
    return moe_epi::router_bwd_impl(grad_out, MOE_EPI_BF16, x, MOE_EPI_BF16, probs, grad_x, grad_probs, rows, hidden,
                                    stream);
}

extern "C" int router_weight_mul_fwd_typed(const void* x, int x_dtype, const float* probs, void* out, int out_dtype,
                                           int64_t rows, int64_t hidden, void* stream) {
    return moe_epi::router_fwd_impl(x, x_dtype, probs, out, out_dtype, rows, hidden, stream);
}

extern "C" int router_weight_mul_bwd_typed(const void* grad_out, int grad_out_dtype, const void* x, int x_dtype,
                                           const float* probs, void* grad_x, float* grad_probs, int64_t rows,
                                           int64_t hidden, void* stream) {
    return moe_epi::router_bwd_impl(grad_out, grad_out_dtype, x, x_dtype, probs, grad_x, grad_probs, rows, hidden,
                                    stream);
}

extern "C" const char* moe_epi_status_string(int status) {
    switch (status) {
        case MOE_EPI_SUCCESS: return "success";
        case MOE_EPI_ERR_NULL_POINTER: return "a required pointer is NULL";
        case MOE_EPI_ERR_BAD_SHAPE: return "bad shape: rows < 0, row width <= 0, or a byte size overflows";
        case MOE_EPI_ERR_BAD_LIMIT: return "limit must be finite and > 0";
        case MOE_EPI_ERR_ALIAS: return "an output overlaps an input or another output";
        case MOE_EPI_ERR_MISALIGNED: return "a pointer is not aligned to its element size";
        case MOE_EPI_ERR_LAUNCH: return "the HIP runtime reported a kernel launch error";
        case MOE_EPI_ERR_BAD_DTYPE: return "unsupported dtype (or dtype pair)";
        default: return "unknown status";
    }
}
