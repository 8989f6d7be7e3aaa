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
// Shape: a token's row is cut into segments of kSegQuads quads (4 consecutive
// elements each; 1024 elements, 4 KiB of float32), one 128-lane block per
// (token, segment) pair, each lane two quads of the segment 128 quads apart,
// so every wavefront-wide quad access covers one contiguous 1 KiB (float32)
// or 512 bytes (16-bit) run. A grid-stride loop takes the pairs past
// kMaxBlocks. The token's slot indices are block-uniform, read 8 at a time
// with unrolled scalar loads, so each routed row's base address lives in
// scalar registers; the local slots of a chunk are kept as a bit mask and
// taken in ascending order, up to kRows rows at a time, whose loads are all
// issued before their adds (which then run in slot order): a token with
// several local rows waits for one memory latency, not one per row. No
// private array is indexed at run time: one that was (a compacted list of the
// chunk's rows) was placed in LDS by the compiler, 8 bytes per lane for each
// of the 1024 lanes the launch bounds allowed, 64 KiB per block. Rows and
// output are streamed once: nontemporal accesses.
//
// Residency. With float32 rows the kernel reads and writes equal byte
// counts, and HBM served that mix fastest with about 24 wavefronts per CU in
// flight: each block reserves kCapLds bytes of LDS that it never touches, so
// that at most kBlocksPerCu blocks share a CU's 160 KiB. With 16-bit rows
// (two thirds of the bytes are writes) the cap made it slower, and a CU holds
// as many blocks as its wavefront slots allow.
//
// Measured at 131072 tokens x 7168 float32 (top-8 of 64 experts, 8 local),
// launched back to back: 1196-1202 us, 78.2-78.6% of HBM peak (one block per
// token: 1277-1301 us, 72.2-73.3%). With a 1 GiB write before every launch,
// bit-identical outputs, in one process per row below: one 896-lane
// block per token (two quads per lane) 73.1-73.6% of HBM peak; 128-lane
// segments with 16 blocks per CU 76.5-76.8%, 14 80.9%, 13 82.6%, 12
// 82.1-82.4%, 11 79.1%, 10 78.7%, 8 74.8%; 64- and 192-lane segments
// 76.6-82.7% and 80.2-81.7% by residency; 256- and 448-lane segments with
// one quad per lane 70.2% and 58.2%; XCD granules of 16 or 64 blocks 65.5%
// and 74.0%. With 16-bit rows: 65.2% one block per token, 69.3% in 128-lane
// segments uncapped, 52.5% capped at 12. At 32768 x 16384 float32: 71.9%
// one block per token, 82.3% in segments. Earlier variants of the one block
// per token shape: one row at a time with 256 lanes x 7 quads 65-67%, a
// persistent grid with the next token's slots prefetched, and a wavefront per
// token, 62-69%; the same kernel on an identity routing (one row per token, in
// order) ran no faster, so the gather itself costs nothing measurable.
#include "epi_common.h"

namespace moe_epi {
namespace {

constexpr int kLanes = 128;        // lanes per block
constexpr int kQuadsPerLane = 2;   // quads of the segment per lane, kLanes apart
constexpr uint32_t kSegQuads = kLanes * kQuadsPerLane;
constexpr int kRows = 4;           // routed rows whose loads are in flight together
constexpr int kSlotChunk = 8;      // slot indices read (unrolled scalar loads) per round
constexpr int64_t kMaxTopK = 1024;  // slots per token accepted (the pages route to a handful)
constexpr int kLdsPerCu = 160 * 1024;  // gfx950
constexpr int kBlocksPerCu = 12;       // float32 rows: resident blocks per CU
constexpr int kCapLds = kLdsPerCu / kBlocksPerCu / 256 * 256;

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

template <int T>
__global__ __launch_bounds__(kLanes) void moe_combine_kernel(const void* __restrict__ expert_out,
                                                             const int32_t* __restrict__ row_of,
                                                             float* __restrict__ out, int64_t rows, int64_t tokens,
                                                             int64_t top_k, int64_t hidden, uint32_t nseg) {
    const uint32_t nq = static_cast<uint32_t>(hidden / 4);
    const int64_t pairs = tokens * static_cast<int64_t>(nseg);
    for (int64_t b = blockIdx.x; b < pairs; b += gridDim.x) {
        const int64_t t = b / nseg;
        const uint32_t c0 = static_cast<uint32_t>(b - t * nseg) * kSegQuads + threadIdx.x;
        const int32_t* slots = row_of + t * top_k;
        f32x4 acc[kQuadsPerLane];
#pragma unroll
        for (int k = 0; k < kQuadsPerLane; ++k) acc[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int64_t j0 = 0; j0 < top_k; j0 += kSlotChunk) {
            // the chunk's rows (block-uniform: scalar loads and registers), local ones flagged in `mask`
            int64_t r[kSlotChunk];
            uint32_t mask = 0;
#pragma unroll
            for (int jj = 0; jj < kSlotChunk; ++jj) {
                r[jj] = -1;
                if (j0 + jj < top_k) {
                    r[jj] = __builtin_amdgcn_readfirstlane(slots[j0 + jj]);
                    if (r[jj] >= 0 && r[jj] < rows) mask |= 1u << jj;
                }
            }
            while (mask) {
                int64_t rr[kRows];
                int n = 0;
#pragma unroll
                for (int q = 0; q < kRows; ++q) {
                    rr[q] = 0;
                    if (mask) {  // the lowest flagged slot, picked by compile-time indices only
                        const int j = __builtin_ctz(mask);
                        mask &= mask - 1;
                        int64_t v = r[0];
#pragma unroll
                        for (int jj = 1; jj < kSlotChunk; ++jj)
                            if (j == jj) v = r[jj];
                        rr[q] = v;
                        n = q + 1;
                    }
                }
                f32x4 v[kRows][kQuadsPerLane];
#pragma unroll
                for (int q = 0; q < kRows; ++q) {
                    if (q >= n) continue;
                    const void* erow = row_at<T>(expert_out, rr[q] * hidden);
#pragma unroll
                    for (int k = 0; k < kQuadsPerLane; ++k) {
                        const uint32_t c = c0 + k * kLanes;
                        v[q][k] = c < nq ? load_quad<T>(erow, 4 * c) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    }
                }
#pragma unroll
                for (int q = 0; q < kRows; ++q)
                    if (q < n)
#pragma unroll
                        for (int k = 0; k < kQuadsPerLane; ++k) acc[k] = acc[k] + v[q][k];
            }
        }
        float* orow = out + t * hidden;
#pragma unroll
        for (int k = 0; k < kQuadsPerLane; ++k) {
            const uint32_t c = c0 + k * kLanes;
            if (c < nq) store_nt16(at<4>(orow, 4 * c), __builtin_bit_cast(u32x4, acc[k]));
        }
    }
}

template <int T>
void launch_combine(const void* eo, const int32_t* row_of, float* out, int64_t rows, int64_t tokens, int64_t top_k,
                    int64_t hidden, hipStream_t st) {
    const int64_t nseg = (hidden / 4 + kSegQuads - 1) / kSegQuads;
    const int lds = T == MOE_EPI_F32 ? kCapLds : 0;
    hipLaunchKernelGGL((moe_combine_kernel<T>), dim3(grid_for_rows(tokens * nseg, 1)), dim3(kLanes), lds, st, eo,
                       row_of, out, rows, tokens, top_k, hidden, static_cast<uint32_t>(nseg));
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
