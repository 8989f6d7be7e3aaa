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
// Kernel shape: as for the SwiGLU kernels, a lane group of G lanes owns a row
// and walks it in 16-byte vectors (8 bf16), V vectors per lane in flight; the
// row sum is a register accumulator reduced with cross-lane shuffles. The
// forward needs no reduction but uses the same row walk, which loads the
// row's probability once and needs no division to find a vector's row.
#include "epi_common.h"

namespace moe_epi {
namespace {

template <int W, int G, int V>
__global__ __launch_bounds__(kBlock) void router_weight_mul_fwd_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ probs, uint16_t* __restrict__ out, int64_t rows,
    int64_t hidden) {
    constexpr int kGroups = kBlock / G;
    const int lane = threadIdx.x & (G - 1);
    const int64_t nvec = hidden / W;
    const int64_t row_step = static_cast<int64_t>(gridDim.x) * kGroups;
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * kGroups + threadIdx.x / G; r < rows; r += row_step) {
        const uint16_t* xr = x + r * hidden;
        uint16_t* orow = out + r * hidden;
        const float p = probs[r];
        for (int64_t c0 = lane; c0 < nvec; c0 += static_cast<int64_t>(G) * V) {
            float v[V][W];
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const int64_t c = c0 + static_cast<int64_t>(k) * G;
                if (c < nvec) Io<W>::load(xr + c * W, v[k]);
            }
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const int64_t c = c0 + static_cast<int64_t>(k) * G;
                if (c < nvec) {
                    float o[W];
#pragma unroll
                    for (int e = 0; e < W; ++e) o[e] = v[k][e] * p;
                    Io<W>::store(orow + c * W, o);
                }
            }
        }
    }
}

template <int W, int G, int V, bool kGradProbs>
__global__ __launch_bounds__(kBlock) void router_weight_mul_bwd_kernel(
    const uint16_t* __restrict__ grad_out, const uint16_t* __restrict__ x, const float* __restrict__ probs,
    uint16_t* __restrict__ grad_x, float* __restrict__ grad_probs, int64_t rows, int64_t hidden) {
    constexpr int kGroups = kBlock / G;
    const int lane = threadIdx.x & (G - 1);
    const int64_t nvec = hidden / W;
    const int64_t row_step = static_cast<int64_t>(gridDim.x) * kGroups;
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * kGroups + threadIdx.x / G; r < rows; r += row_step) {
        const uint16_t* gr = grad_out + r * hidden;
        const uint16_t* xr = x + r * hidden;
        uint16_t* gxr = grad_x + r * hidden;
        const float p = probs[r];
        float acc = 0.0f;
        for (int64_t c0 = lane; c0 < nvec; c0 += static_cast<int64_t>(G) * V) {
            float g[V][W], xv[V][W];
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const int64_t c = c0 + static_cast<int64_t>(k) * G;
                if (c < nvec) {
                    Io<W>::load(gr + c * W, g[k]);
                    if (kGradProbs) Io<W>::load(xr + c * W, xv[k]);
                }
            }
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const int64_t c = c0 + static_cast<int64_t>(k) * G;
                if (c < nvec) {
                    float o[W];
#pragma unroll
                    for (int e = 0; e < W; ++e) {
                        o[e] = g[k][e] * p;
                        // a product of two bf16 values is exact in fp32
                        if (kGradProbs) acc = __fmaf_rn(g[k][e], xv[k][e], acc);
                    }
                    Io<W>::store(gxr + c * W, o);
                }
            }
        }
        if (kGradProbs) {
            acc = group_sum<G>(acc);
            if (lane == 0) grad_probs[r] = acc;
        }
    }
}

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
void launch_fwd(const uint16_t* x, const float* probs, uint16_t* out, int64_t rows, int64_t hidden, hipStream_t st) {
    const unsigned grid = grid_for_rows(rows, kBlock / G, kMaxBlocks);
    hipLaunchKernelGGL((router_weight_mul_fwd_kernel<W, G, V>), dim3(grid), dim3(kBlock), 0, st, x, probs, out, rows,
                       hidden);
}

template <int W, int G, int V>
void launch_bwd(const uint16_t* go, const uint16_t* x, const float* probs, uint16_t* gx, float* gp, int64_t rows,
                int64_t hidden, hipStream_t st) {
    const unsigned grid = grid_for_rows(rows, kBlock / G, kMaxBlocks);
    if (gp)
        hipLaunchKernelGGL((router_weight_mul_bwd_kernel<W, G, V, true>), dim3(grid), dim3(kBlock), 0, st, go, x,
                           probs, gx, gp, rows, hidden);
    else
        hipLaunchKernelGGL((router_weight_mul_bwd_kernel<W, G, V, false>), dim3(grid), dim3(kBlock), 0, st, go, x,
                           probs, gx, gp, rows, hidden);
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
        const Shape sh = pick_shape(hidden / 8);
        MOE_EPI_DISPATCH_SHAPE(sh, launch_fwd, x, probs, out, rows, hidden, s);
    } else {
        launch_fwd<1, 64, 4>(x, probs, out, rows, hidden, s);
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
        const Shape sh = pick_shape(hidden / 8);
        MOE_EPI_DISPATCH_SHAPE(sh, launch_bwd, grad_out, x, probs, grad_x, grad_probs, rows, hidden, s);
    } else {
        launch_bwd<1, 64, 4>(grad_out, x, probs, grad_x, grad_probs, rows, hidden, s);
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
