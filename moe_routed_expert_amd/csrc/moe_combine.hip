// Combine of the routed rows back into tokens (gfx950).
//
// Pages: "nemo_automodel.components.moe.quantized_experts",
// GroupedExpertsMXFP4.forward: the local experts' contribution to each token
// is an fp32 [tokens, hidden] tensor, the sum of the token's top-k routed
// rows that belong to this rank's experts (the other slots add nothing);
// "nemo_automodel.components.moe.optimized_ops", _apply_router_weight_fp32:
// the routed rows come out of the router-weight multiply in fp32 so that this
// sum is taken in fp32.
//
// For token t: out[t, :] = +0 + expert_out[row_of[t, 0], :] + ... +
// expert_out[row_of[t, top_k - 1], :], binary32 adds in ascending slot order,
// a slot whose row index is outside [0, rows) skipped (not local, or absent).
// Every element of out gets the same sequence of binary32 operations as this
// definition, so the result is bit-exact whatever the launch shape.
//
// Shape: one block per token (a grid-stride loop past kMaxBlocks tokens). The
// token's slot indices are block-uniform, so they are read with scalar loads
// and each routed row's base address lives in scalar registers. A lane owns V
// quads (4 consecutive elements) of the row per pass, 256 lanes per block: one
// pass covers V * 1024 elements (hidden 7168: V = 7, one pass). Per pass the
// lane issues the V loads of a row before the adds, so V independent 16-byte
// (float32) or 8-byte (16-bit) loads are in flight per lane. A wavefront's
// quad access covers 1 KiB of float32 or 512 bytes of 16-bit data
// contiguously. Rows and output are streamed once: nontemporal accesses.
#include "epi_common.h"

namespace moe_epi {
namespace {

constexpr int kCombineThreads = 256;
constexpr int kMaxQuadsPerLane = 8;
constexpr int64_t kMaxTopK = 1024;  // slots per token accepted (the pages route to a handful)

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int T>
__device__ __forceinline__ f32x4 load_quad(const void* row, uint32_t e) {
    if constexpr (T == MOE_EPI_F32) {
        return __builtin_bit_cast(f32x4, load_nt16(at<4>(row, e)));
    } else {
        const u32x2 w = load_nt8(at<2>(row, e));
        float f[8];
        Elem<T>::unpack(u32x4{w[0], w[1], 0u, 0u}, f);
        return f32x4{f[0], f[1], f[2], f[3]};
    }
}

template <int T, int V>
__global__ __launch_bounds__(kCombineThreads) void moe_combine_kernel(const void* __restrict__ expert_out,
                                                                      const int32_t* __restrict__ row_of,
                                                                      float* __restrict__ out, int64_t rows,
                                                                      int64_t tokens, int64_t top_k, int64_t hidden) {
    const uint32_t nq = static_cast<uint32_t>(hidden / 4);
    const uint32_t lane = threadIdx.x;
    for (int64_t t = blockIdx.x; t < tokens; t += gridDim.x) {
        const int32_t* slots = row_of + t * top_k;
        float* orow = out + t * hidden;
        for (uint32_t c0 = lane; c0 < nq; c0 += kCombineThreads * V) {
            f32x4 acc[V];
#pragma unroll
            for (int k = 0; k < V; ++k) acc[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            for (int64_t j = 0; j < top_k; ++j) {
                const int64_t r = __builtin_amdgcn_readfirstlane(slots[j]);
                if (r < 0 || r >= rows) continue;
                const void* erow = row_at<T>(expert_out, r * hidden);
                f32x4 v[V];
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const uint32_t c = c0 + k * kCombineThreads;
                    v[k] = c < nq ? load_quad<T>(erow, 4 * c) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                }
#pragma unroll
                for (int k = 0; k < V; ++k) acc[k] = acc[k] + v[k];
            }
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const uint32_t c = c0 + k * kCombineThreads;
                if (c < nq) store_nt16(at<4>(orow, 4 * c), __builtin_bit_cast(u32x4, acc[k]));
            }
        }
    }
}

template <int T, int V>
void launch_combine_v(const void* eo, const int32_t* row_of, float* out, int64_t rows, int64_t tokens, int64_t top_k,
                      int64_t hidden, hipStream_t st) {
    hipLaunchKernelGGL((moe_combine_kernel<T, V>), dim3(grid_for_rows(tokens, 1)), dim3(kCombineThreads), 0, st, eo,
                       row_of, out, rows, tokens, top_k, hidden);
}

template <int T>
void launch_combine(const void* eo, const int32_t* row_of, float* out, int64_t rows, int64_t tokens, int64_t top_k,
                    int64_t hidden, hipStream_t st) {
    // quads per lane: enough for one pass over the row, at most kMaxQuadsPerLane
    const int64_t per_lane = (hidden / 4 + kCombineThreads - 1) / kCombineThreads;
    switch (per_lane <= 1 ? 1 : (per_lane >= kMaxQuadsPerLane ? kMaxQuadsPerLane : per_lane)) {
        case 1: return launch_combine_v<T, 1>(eo, row_of, out, rows, tokens, top_k, hidden, st);
        case 2: return launch_combine_v<T, 2>(eo, row_of, out, rows, tokens, top_k, hidden, st);
        case 3: return launch_combine_v<T, 3>(eo, row_of, out, rows, tokens, top_k, hidden, st);
        case 4: return launch_combine_v<T, 4>(eo, row_of, out, rows, tokens, top_k, hidden, st);
        case 5: return launch_combine_v<T, 5>(eo, row_of, out, rows, tokens, top_k, hidden, st);
        case 6: return launch_combine_v<T, 6>(eo, row_of, out, rows, tokens, top_k, hidden, st);
        case 7: return launch_combine_v<T, 7>(eo, row_of, out, rows, tokens, top_k, hidden, st);
        default: return launch_combine_v<T, 8>(eo, row_of, out, rows, tokens, top_k, hidden, st);
    }
}

}  // namespace
}  // namespace moe_epi

using namespace moe_epi;

extern "C" int moe_combine_fwd(const void* expert_out, int eo_dtype, const int32_t* row_of, float* out, int64_t rows,
                               int64_t tokens, int64_t top_k, int64_t hidden, void* stream) {
    if (!dtype_ok(eo_dtype)) return MOE_EPI_ERR_BAD_DTYPE;
    if (rows < 0 || tokens < 0 || top_k < 1 || top_k > kMaxTopK || hidden <= 0 || hidden % 8 != 0 ||
        !row_fits_u32_offsets(hidden, 4))
        return MOE_EPI_ERR_BAD_SHAPE;
    const int eb = elem_bytes(eo_dtype);
    int64_t eob = 0, rob, ob;
    if ((rows > 0 && !bytes_ok(rows, hidden, eb, &eob)) || !bytes_ok(tokens, top_k, 4, &rob) ||
        !bytes_ok(tokens, hidden, 4, &ob))
        return MOE_EPI_ERR_BAD_SHAPE;
    if (tokens == 0) return MOE_EPI_SUCCESS;
    if ((rows > 0 && !expert_out) || !row_of || !out) return MOE_EPI_ERR_NULL_POINTER;
    if (!aligned(expert_out, 16) || !aligned(out, 16) || !aligned(row_of, 4)) return MOE_EPI_ERR_MISALIGNED;
    const Range ro = range_of(out, ob);
    if (overlaps(ro, range_of(expert_out, eob)) || overlaps(ro, range_of(row_of, rob))) return MOE_EPI_ERR_ALIAS;
    (void)hipGetLastError();
    const hipStream_t st = as_stream(stream);
    switch (eo_dtype) {
        case MOE_EPI_BF16: launch_combine<MOE_EPI_BF16>(expert_out, row_of, out, rows, tokens, top_k, hidden, st); break;
        case MOE_EPI_F16: launch_combine<MOE_EPI_F16>(expert_out, row_of, out, rows, tokens, top_k, hidden, st); break;
        default: launch_combine<MOE_EPI_F32>(expert_out, row_of, out, rows, tokens, top_k, hidden, st); break;
    }
    return launch_status();
}
