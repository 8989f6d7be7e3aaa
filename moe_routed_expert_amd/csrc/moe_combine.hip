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
// Shape: one block per token (a grid-stride loop past kMaxBlocks tokens), B
// lanes that own V quads (4 consecutive elements) each per pass over the row,
// B * V about the row's quad count (hidden 7168: B = 896, V = 2, one pass). The
// token's slot indices are block-uniform, read 8 at a time with unrolled scalar
// loads (a loop that reads one index per iteration was compiled to vector
// loads, each waited for in turn: 65% of peak instead of 73%), so each routed
// row's base address lives in scalar registers. Rows are taken kRows at
// a time: the loads of up to kRows rows are all issued before their adds
// (which then run in slot order), so a token with several local rows waits
// for one memory latency, not one per row. A wavefront's quad access covers
// 1 KiB of float32 or 512 bytes of 16-bit data contiguously. Rows and output
// are streamed once: nontemporal accesses.
//
// Measured at 131072 tokens x 7168 float32 (top-8 of 64 experts, 8 local):
// one row at a time with 256 lanes x 7 quads ran at 65-67% of HBM peak; three
// rows at a time 70-71%; with 896 lanes x 2 quads 73%. Limiting the resident
// blocks (by LDS, to 2-8 per CU) changed nothing; a persistent grid with the
// next token's slots prefetched, and a wavefront per token, ran at 62-69%. The
// same kernel on an identity routing (one row per token, in order) ran no
// faster, so the gather itself costs nothing measurable.
#include "epi_common.h"

namespace moe_epi {
namespace {

constexpr int kMaxThreads = 1024;
constexpr int kRows = 3;       // routed rows whose loads are in flight together
constexpr int kSlotChunk = 8;  // slot indices read (unrolled scalar loads) per round
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
__global__ __launch_bounds__(kMaxThreads) void moe_combine_kernel(const void* __restrict__ expert_out,
                                                                  const int32_t* __restrict__ row_of,
                                                                  float* __restrict__ out, int64_t rows,
                                                                  int64_t tokens, int64_t top_k, int64_t hidden) {
    const uint32_t nq = static_cast<uint32_t>(hidden / 4);
    const uint32_t lane = threadIdx.x, nb = blockDim.x;
    for (int64_t t = blockIdx.x; t < tokens; t += gridDim.x) {
        const int32_t* slots = row_of + t * top_k;
        float* orow = out + t * hidden;
        for (uint32_t c0 = lane; c0 < nq; c0 += nb * V) {
            f32x4 acc[V];
#pragma unroll
            for (int k = 0; k < V; ++k) acc[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            for (int64_t j0 = 0; j0 < top_k; j0 += kSlotChunk) {
                // the chunk's local rows, in slot order (block-uniform: scalar loads and registers)
                int64_t list[kSlotChunk];
                int n = 0;
#pragma unroll
                for (int jj = 0; jj < kSlotChunk; ++jj) {
                    if (j0 + jj < top_k) {
                        const int64_t r = __builtin_amdgcn_readfirstlane(slots[j0 + jj]);
                        if (r >= 0 && r < rows) list[n++] = r;
                    }
                }
                for (int i = 0; i < n; i += kRows) {
                    f32x4 v[kRows][V];
#pragma unroll
                    for (int q = 0; q < kRows; ++q) {
                        if (i + q >= n) continue;
                        const void* erow = row_at<T>(expert_out, list[i + q] * hidden);
#pragma unroll
                        for (int k = 0; k < V; ++k) {
                            const uint32_t c = c0 + k * nb;
                            v[q][k] = c < nq ? load_quad<T>(erow, 4 * c) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                        }
                    }
#pragma unroll
                    for (int q = 0; q < kRows; ++q)
                        if (i + q < n)
#pragma unroll
                            for (int k = 0; k < V; ++k) acc[k] = acc[k] + v[q][k];
                }
            }
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const uint32_t c = c0 + k * nb;
                if (c < nq) store_nt16(at<4>(orow, 4 * c), __builtin_bit_cast(u32x4, acc[k]));
            }
        }
    }
}

// Quads per lane and lanes per block for a row of nq quads: V = 1, 2 or 4 and
// B a multiple of 64 with B * V >= nq where that fits in one block, else
// kMaxThreads x 4 and several passes.
template <int T>
void launch_combine(const void* eo, const int32_t* row_of, float* out, int64_t rows, int64_t tokens, int64_t top_k,
                    int64_t hidden, hipStream_t st) {
    const int64_t nq = hidden / 4;
    const int v = nq <= kMaxThreads ? 1 : (nq <= 2 * kMaxThreads ? 2 : 4);
    int64_t b = (nq + v - 1) / v;
    b = (b + 63) / 64 * 64;
    if (b > kMaxThreads) b = kMaxThreads;
    const dim3 grid(grid_for_rows(tokens, 1)), block(static_cast<unsigned>(b));
    if (v == 1)
        hipLaunchKernelGGL((moe_combine_kernel<T, 1>), grid, block, 0, st, eo, row_of, out, rows, tokens, top_k, hidden);
    else if (v == 2)
        hipLaunchKernelGGL((moe_combine_kernel<T, 2>), grid, block, 0, st, eo, row_of, out, rows, tokens, top_k, hidden);
    else
        hipLaunchKernelGGL((moe_combine_kernel<T, 4>), grid, block, 0, st, eo, row_of, out, rows, tokens, top_k, hidden);
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
