// fp32 router-weight multiply: forward and backward for gfx950.
//
// Operation (page "nemo_automodel.components.moe.optimized_ops", entries
// _RouterWeightMulFunction, _rw_fwd_core, _rw_bwd_x_core, _rw_bwd_probs_core):
// on the expert down-projection output x [tokens, hidden] with one fp32
// routing probability per row,
//   out        = bf16(fp32(x) * p)                 (bitwise equal to the eager multiply)
//   grad_x     = bf16(fp32(grad_out) * p)
//   grad_probs = sum_k fp32(grad_out) * fp32(x)     (fp32)
// The page computes the two gradients with two cores, i.e. two passes over
// grad_out; here both come out of one pass (grad_out and x read once).
//
// Kernel shape: as for the SwiGLU kernels, a group of G lanes owns a row and
// walks it in 16-byte nontemporal vectors (8 bf16), V vectors per lane in
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
// of a block runs the same iterations (row_sum may hold a barrier).
template <int G, int V, int B>
__global__ __launch_bounds__(B) void router_weight_mul_fwd_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ probs, uint16_t* __restrict__ out, int64_t rows,
    int64_t hidden) {
    constexpr int kRows = B / G;
    const int lane = threadIdx.x % G;
    const int64_t nvec = hidden / 8;
    for (int64_t rb = static_cast<int64_t>(blockIdx.x) * kRows; rb < rows;
         rb += static_cast<int64_t>(gridDim.x) * kRows) {
        const int64_t r = rb + threadIdx.x / G;
        if (r >= rows) continue;
        const uint16_t* xr = x + r * hidden;
        uint16_t* orow = out + r * hidden;
        const float p = probs[r];
        for (int64_t c0 = lane; c0 < nvec; c0 += static_cast<int64_t>(G) * V) {
            u32x4 v[V];
#pragma unroll
            for (int k = 0; k < V; ++k)
                if (c0 + k * G < nvec) v[k] = load_stream(xr + (c0 + k * G) * 8);
#pragma unroll
            for (int k = 0; k < V; ++k) {
                if (c0 + k * G < nvec) {
                    u32x4 o;
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(bf16_lo(v[k][i]) * p, bf16_hi(v[k][i]) * p);
                    store_stream(orow + (c0 + k * G) * 8, o);
                }
            }
        }
    }
}

template <int G, int V, int B, bool kGradProbs>
__global__ __launch_bounds__(B) void router_weight_mul_bwd_kernel(
    const uint16_t* __restrict__ grad_out, const uint16_t* __restrict__ x, const float* __restrict__ probs,
    uint16_t* __restrict__ grad_x, float* __restrict__ grad_probs, int64_t rows, int64_t hidden) {
    constexpr int kRows = B / G;
    __shared__ float part[B / 64 > 0 ? B / 64 : 1];
    const int lane = threadIdx.x % G;
    const int64_t nvec = hidden / 8;
    for (int64_t rb = static_cast<int64_t>(blockIdx.x) * kRows; rb < rows;
         rb += static_cast<int64_t>(gridDim.x) * kRows) {
        const int64_t r = rb + threadIdx.x / G;
        float acc = 0.0f;
        if (r < rows) {
            const uint16_t* gr = grad_out + r * hidden;
            const uint16_t* xr = x + r * hidden;
            uint16_t* gxr = grad_x + r * hidden;
            const float p = probs[r];
            for (int64_t c0 = lane; c0 < nvec; c0 += static_cast<int64_t>(G) * V) {
                u32x4 g[V], xv[V];
#pragma unroll
                for (int k = 0; k < V; ++k)
                    if (c0 + k * G < nvec) g[k] = load_stream(gr + (c0 + k * G) * 8);
                if (kGradProbs) {
#pragma unroll
                    for (int k = 0; k < V; ++k)
                        if (c0 + k * G < nvec) xv[k] = load_stream(xr + (c0 + k * G) * 8);
                }
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    if (c0 + k * G < nvec) {
                        u32x4 o;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float g0 = bf16_lo(g[k][i]), g1 = bf16_hi(g[k][i]);
                            o[i] = pack_bf16x2(g0 * p, g1 * p);
                            // a product of two bf16 values is exact in fp32
                            if (kGradProbs) {
                                acc = __fmaf_rn(g0, bf16_lo(xv[k][i]), acc);
                                acc = __fmaf_rn(g1, bf16_hi(xv[k][i]), acc);
                            }
                        }
                        store_stream(gxr + (c0 + k * G) * 8, o);
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

// per-element kernels (any hidden, 2-byte aligned tensors)
__global__ __launch_bounds__(kBlock) void router_weight_mul_fwd_scalar_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ probs, uint16_t* __restrict__ out, int64_t rows,
    int64_t hidden) {
    constexpr int kRows = kBlock / 64;
    const int lane = threadIdx.x % 64;
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * kRows + threadIdx.x / 64; r < rows;
         r += static_cast<int64_t>(gridDim.x) * kRows) {
        const float p = probs[r];
        for (int64_t k = lane; k < hidden; k += 64) out[r * hidden + k] = to_bf16(bf16_at(x + r * hidden + k) * p);
    }
}

template <bool kGradProbs>
__global__ __launch_bounds__(kBlock) void router_weight_mul_bwd_scalar_kernel(
    const uint16_t* __restrict__ grad_out, const uint16_t* __restrict__ x, const float* __restrict__ probs,
    uint16_t* __restrict__ grad_x, float* __restrict__ grad_probs, int64_t rows, int64_t hidden) {
    constexpr int kRows = kBlock / 64;
    const int lane = threadIdx.x % 64;
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * kRows + threadIdx.x / 64; r < rows;
         r += static_cast<int64_t>(gridDim.x) * kRows) {
        const float p = probs[r];
        float acc = 0.0f;
        for (int64_t k = lane; k < hidden; k += 64) {
            const float g = bf16_at(grad_out + r * hidden + k);
            grad_x[r * hidden + k] = to_bf16(g * p);
            if (kGradProbs) acc = __fmaf_rn(g, bf16_at(x + r * hidden + k), acc);
        }
        if (kGradProbs) {
            acc = group_sum<64>(acc);
            if (lane == 0) grad_probs[r] = acc;
        }
    }
}

// Shapes (measured on MI355X at 65536 x 7168; nontemporal 16-byte accesses):
//   forward:  2 wavefronts per row, 256-thread blocks, up to 16 vectors per
//             lane per pass (7168: 7 per lane, the whole row in one pass);
//   backward: 2 vectors per lane and as many wavefronts per row as that needs
//             (7168: 7 wavefronts), two rows per block where that fits in 1024
//             threads. Against one wavefront per row (14 vectors per lane) the
//             forward ran 2% and the backward 8% faster: a row's loads are
//             issued from several SIMDs at once.
template <int G, int V, int B>
void launch_fwd(const uint16_t* x, const float* probs, uint16_t* out, int64_t rows, int64_t hidden, hipStream_t st) {
    hipLaunchKernelGGL((router_weight_mul_fwd_kernel<G, V, B>), dim3(grid_for_rows(rows, B / G)), dim3(B), 0, st, x,
                       probs, out, rows, hidden);
}

template <int G, int V, int B>
void launch_bwd(const uint16_t* go, const uint16_t* x, const float* probs, uint16_t* gx, float* gp, int64_t rows,
                int64_t hidden, hipStream_t st) {
    const dim3 grid(grid_for_rows(rows, B / G));
    if (gp)
        hipLaunchKernelGGL((router_weight_mul_bwd_kernel<G, V, B, true>), grid, dim3(B), 0, st, go, x, probs, gx, gp,
                           rows, hidden);
    else
        hipLaunchKernelGGL((router_weight_mul_bwd_kernel<G, V, B, false>), grid, dim3(B), 0, st, go, x, probs, gx, gp,
                           rows, hidden);
}

void dispatch_fwd(const uint16_t* x, const float* probs, uint16_t* out, int64_t rows, int64_t hidden,
                  hipStream_t st) {
    const int64_t nvec = hidden / 8;
    if (nvec < 64) {
        switch (small_group(nvec)) {
            case 8: return launch_fwd<8, 1, 256>(x, probs, out, rows, hidden, st);
            case 16: return launch_fwd<16, 1, 256>(x, probs, out, rows, hidden, st);
            default: return launch_fwd<32, 1, 256>(x, probs, out, rows, hidden, st);
        }
    }
    if (nvec < 128) return launch_fwd<64, 2, 256>(x, probs, out, rows, hidden, st);
    switch (ceil_div(nvec, 128)) {  // vectors per lane with 128 lanes per row
        case 1: return launch_fwd<128, 1, 256>(x, probs, out, rows, hidden, st);
        case 2: return launch_fwd<128, 2, 256>(x, probs, out, rows, hidden, st);
        case 3: return launch_fwd<128, 3, 256>(x, probs, out, rows, hidden, st);
        case 4: return launch_fwd<128, 4, 256>(x, probs, out, rows, hidden, st);
        case 5: return launch_fwd<128, 5, 256>(x, probs, out, rows, hidden, st);
        case 6: return launch_fwd<128, 6, 256>(x, probs, out, rows, hidden, st);
        case 7: return launch_fwd<128, 7, 256>(x, probs, out, rows, hidden, st);
        case 8: return launch_fwd<128, 8, 256>(x, probs, out, rows, hidden, st);
        case 9: case 10: return launch_fwd<128, 10, 256>(x, probs, out, rows, hidden, st);
        case 11: case 12: return launch_fwd<128, 12, 256>(x, probs, out, rows, hidden, st);
        case 13: case 14: return launch_fwd<128, 14, 256>(x, probs, out, rows, hidden, st);
        default: return launch_fwd<128, 16, 256>(x, probs, out, rows, hidden, st);
    }
}

void dispatch_bwd(const uint16_t* go, const uint16_t* x, const float* probs, uint16_t* gx, float* gp, int64_t rows,
                  int64_t hidden, hipStream_t st) {
    const int64_t nvec = hidden / 8;
    if (nvec < 64) {
        switch (small_group(nvec)) {
            case 8: return launch_bwd<8, 1, 256>(go, x, probs, gx, gp, rows, hidden, st);
            case 16: return launch_bwd<16, 1, 256>(go, x, probs, gx, gp, rows, hidden, st);
            default: return launch_bwd<32, 1, 256>(go, x, probs, gx, gp, rows, hidden, st);
        }
    }
    switch (ceil_div(nvec, 128)) {  // wavefronts per row with 2 vectors per lane
        case 1: return launch_bwd<64, 2, 128>(go, x, probs, gx, gp, rows, hidden, st);
        case 2: return launch_bwd<128, 2, 256>(go, x, probs, gx, gp, rows, hidden, st);
        case 3: return launch_bwd<192, 2, 384>(go, x, probs, gx, gp, rows, hidden, st);
        case 4: return launch_bwd<256, 2, 512>(go, x, probs, gx, gp, rows, hidden, st);
        case 5: return launch_bwd<320, 2, 640>(go, x, probs, gx, gp, rows, hidden, st);
        case 6: return launch_bwd<384, 2, 768>(go, x, probs, gx, gp, rows, hidden, st);
        case 7: return launch_bwd<448, 2, 896>(go, x, probs, gx, gp, rows, hidden, st);
        case 8: return launch_bwd<512, 2, 1024>(go, x, probs, gx, gp, rows, hidden, st);
        case 9: return launch_bwd<576, 2, 576>(go, x, probs, gx, gp, rows, hidden, st);
        case 10: return launch_bwd<640, 2, 640>(go, x, probs, gx, gp, rows, hidden, st);
        case 11: return launch_bwd<704, 2, 704>(go, x, probs, gx, gp, rows, hidden, st);
        case 12: return launch_bwd<768, 2, 768>(go, x, probs, gx, gp, rows, hidden, st);
        case 13: return launch_bwd<832, 2, 832>(go, x, probs, gx, gp, rows, hidden, st);
        case 14: return launch_bwd<896, 2, 896>(go, x, probs, gx, gp, rows, hidden, st);
        case 15: return launch_bwd<960, 2, 960>(go, x, probs, gx, gp, rows, hidden, st);
        default: return launch_bwd<1024, 2, 1024>(go, x, probs, gx, gp, rows, hidden, st);  // wider rows: passes
    }
}

int check_router(int64_t rows, int64_t hidden, int64_t* h_bytes, int64_t* p_bytes) {
    if (rows < 0 || hidden <= 0) return MOE_EPI_ERR_BAD_SHAPE;
    if (!bytes_ok(rows, hidden, 2, h_bytes) || !bytes_ok(rows, 1, 4, p_bytes)) return MOE_EPI_ERR_BAD_SHAPE;
    return MOE_EPI_SUCCESS;
}

}  // namespace
}  // namespace moe_epi

extern "C" int router_weight_mul_fwd(const uint16_t* x, const float* probs, uint16_t* out, int64_t rows,
                                     int64_t hidden, void* stream) {
    using namespace moe_epi;
    int64_t hb, pb;
    int st = check_router(rows, hidden, &hb, &pb);
    if (st != MOE_EPI_SUCCESS) return st;
    if (rows == 0) return MOE_EPI_SUCCESS;
    if (!x || !probs || !out) return MOE_EPI_ERR_NULL_POINTER;
    if (!aligned(x, 2) || !aligned(out, 2) || !aligned(probs, 4)) return MOE_EPI_ERR_MISALIGNED;
    const Range rx = range_of(x, hb), rp = range_of(probs, pb), ro = range_of(out, hb);
    if (overlaps(ro, rx) || overlaps(ro, rp)) return MOE_EPI_ERR_ALIAS;

    hipStream_t s = as_stream(stream);
    (void)hipGetLastError();
    if (hidden % 8 == 0 && aligned(x, 16) && aligned(out, 16)) {
        dispatch_fwd(x, probs, out, rows, hidden, s);
    } else {
        hipLaunchKernelGGL(router_weight_mul_fwd_scalar_kernel, dim3(grid_for_rows(rows, kBlock / 64)), dim3(kBlock),
                           0, s, x, probs, out, rows, hidden);
    }
    return launch_status();
}

extern "C" int router_weight_mul_bwd(const uint16_t* grad_out, const uint16_t* x, const float* probs,
                                     uint16_t* grad_x, float* grad_probs, int64_t rows, int64_t hidden,
                                     void* stream) {
    using namespace moe_epi;
    int64_t hb, pb;
    int st = check_router(rows, hidden, &hb, &pb);
    if (st != MOE_EPI_SUCCESS) return st;
    if (rows == 0) return MOE_EPI_SUCCESS;
    if (!grad_out || !probs || !grad_x || (grad_probs && !x)) return MOE_EPI_ERR_NULL_POINTER;
    if (!grad_probs) x = nullptr;  // x is only read for the probability gradient
    if (!aligned(grad_out, 2) || !aligned(grad_x, 2) || !aligned(probs, 4) || (x && !aligned(x, 2)) ||
        (grad_probs && !aligned(grad_probs, 4)))
        return MOE_EPI_ERR_MISALIGNED;
    const Range rgo = range_of(grad_out, hb), rx = range_of(x, x ? hb : 0), rp = range_of(probs, pb);
    const Range rgx = range_of(grad_x, hb), rgp = range_of(grad_probs, grad_probs ? pb : 0);
    if (overlaps(rgx, rgo) || overlaps(rgx, rx) || overlaps(rgx, rp) || overlaps(rgp, rgo) || overlaps(rgp, rx) ||
        overlaps(rgp, rp) || overlaps(rgp, rgx))
        return MOE_EPI_ERR_ALIAS;

    hipStream_t s = as_stream(stream);
    (void)hipGetLastError();
    if (hidden % 8 == 0 && aligned(grad_out, 16) && aligned(grad_x, 16) && (!x || aligned(x, 16))) {
        dispatch_bwd(grad_out, x, probs, grad_x, grad_probs, rows, hidden, s);
    } else {
        const dim3 grid(grid_for_rows(rows, kBlock / 64));
        if (grad_probs)
            hipLaunchKernelGGL(router_weight_mul_bwd_scalar_kernel<true>, grid, dim3(kBlock), 0, s, grad_out, x,
                               probs, grad_x, grad_probs, rows, hidden);
        else
            hipLaunchKernelGGL(router_weight_mul_bwd_scalar_kernel<false>, grid, dim3(kBlock), 0, s, grad_out, x,
                               probs, grad_x, grad_probs, rows, hidden);
    }
    return launch_status();
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
        default: return "unknown status";
    }
}
