// Grouped GEMMs of the routed experts for gfx950 (bf16 MFMA, fp32
// accumulation), one kernel template with two epilogues: the gate_up GEMM with
// the clamped SwiGLU x probability epilogue, and the down projection with the
// router-weight multiply epilogue (bf16 or fp32 output).
//
// Operation (gate_up). Pages: "nemo_automodel.components.moe.mok_experts" (the routed
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
// Operation (down). Pages: "nemo_automodel.components.moe.mok_experts" (the
// routed down weights are contiguous bf16 [local_experts, hidden,
// expert_intermediate]); the grouped product as above;
// "nemo_automodel.components.moe.optimized_ops", _apply_router_weight_fp32
// (the product times the permuted probability in fp32, cast to the output
// dtype). For a row t of local expert e:
//   out2[t, n] = bf16(sum_i h[t, i] * w_down[e, n, i])   (fp32 accumulation)
//   out[t, n]  = out_dtype(float(out2[t, n]) * p[t])
// The block's two weight tiles are then two consecutive 128-column ranges of
// w_down[e], so a block covers 256 output columns.
//
// Kernel shape (the launched configurations, ProdGateUp and ProdDown below):
//   * A block computes a 256-token x 128-column tile of gate and the same
//     tile of up (so each output's gate and up sit in the same lane), with
//     eight wavefronts (4 x 2) of 64 x 64 each: 2 x 2 v_mfma_f32_32x32x16_bf16
//     tiles for gate and 2 x 2 for up, 128 fp32 accumulators per lane, two
//     wavefronts per SIMD, one block per CU (128 KiB of LDS).
//   * Operands go from global memory straight into LDS (global_load_lds_dwordx4),
//     K steps of 64, two LDS stages: the next step's loads are in flight while
//     this step's MFMAs run, with no registers spent on staging. Tiles are not
//     padded (a wavefront's load fills 1 KiB contiguously); an XOR swizzle of
//     each row's 16-byte chunks keeps the fragment reads conflict-free.
//   * Within a K step, the next 16-wide sub-step's fragments are read from LDS
//     while the current one's MFMAs run, one read placed after each MFMA. One
//     barrier per K step, before the last sub-step, a bare s_barrier after
//     explicit waits (a __syncthreads() fence would also wait for the loads
//     still in flight); the loads of the step after next and the next step's
//     first fragments are issued while the last sub-step's MFMAs run, one
//     MFMA, one load, one read at a time, the loads in buffer form.
//   * Tiles never straddle experts: each block finds its expert and row range
//     from offs on the device (no host copy of offs), so a grid sized for
//     the worst case, ceil(tokens / 256) + experts row tiles, covers any split.
//   * Tile order: tiles are visited in groups of row tiles (4 for gate_up, 32
//     for the down projection), the row tile changing fastest, so that the
//     blocks running together on one XCD share both their A tiles and their
//     weight tiles in that XCD's L2. The hardware hands consecutive block ids
//     to the 8 XCDs in turn, and the kernel keeps that placement: all XCDs
//     then work on neighbouring tiles of the same expert, and their L2 misses
//     on its weights and activations hit the shared Infinity Cache. Giving
//     each XCD a contiguous range of tiles instead puts the XCDs on different
//     experts: gate_up 1061 TFLOP/s against 1107, the down projection 1008
//     against 1023.
//   * Epilogue: accumulators are rounded to bf16, the SwiGLU is applied, and
//     each output tile is staged through LDS so that global stores are
//     16-byte, row-contiguous accesses.
// Measured at 131072 x 7168 x 2048 with 8 experts (every configuration gives
// bit-identical results, each output being accumulated in the same order):
// register-staged loads with padded LDS ran at 746-918 TFLOP/s over 22 tile
// shapes, deeper load pipelines and fragment pipelining at up to 953, the
// same tiles with one barrier per step at 941-965, and this loop at 1040-1060
// (MFMA busy 54% of cycles, LDS 21%, bank conflicts 0.8% of LDS cycles) with
// an XCD-contiguous block order, 1090-1108 with the round-robin one, and
// 1174-1202 with the last sub-step's loads interleaved between its MFMAs.
// Variants that did not help: K steps of 32 with 3-5 stages (850-912), two
// 128 x 128 blocks per CU (870-890), other read placements (1007-1049), a
// branch-free unrolled loop (1022-1032), an L2 prefetch two to four steps
// ahead (930), A tiles three stages deep (929), four wavefronts of 128-row
// tiles (950), raised wave priority around the MFMAs (997), a ping-pong of
// two wavefront groups alternating fragment-read and MFMA phases (885-925),
// accumulators in AGPRs (no change), the next step's loads spread between
// the MFMAs of the current one (982-990), register-staged loads instead of
// direct-to-LDS ones (775-823), A tiles three stages deep (962). Timing-only
// copies before the interleave: MFMAs, barriers and epilogue alone 1677, plus
// the fragment reads 1475, plus loads that all hit L2 1198, as launched 1100;
// the loads not waited for at the barrier: no change. The shader clock averages about
// 1.58 GHz in this kernel (busy cycles per XCD over the dispatch time; 1.74
// before the loads were interleaved: the part is power-limited here), so
// 2.5 PFLOP/s at 2.4 GHz is about 1.65 PFLOP/s at the clock it runs at.
#include "epi_common.h"
#include "grouped_map.h"
#include "swiglu_math.h"

namespace moe_epi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

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

// ---- the kernel -------------------------------------------------------------------
//
// Global loads write straight into LDS (global_load_lds_dwordx4: each lane's
// 16 bytes land at the wavefront's LDS base + 16 * lane), one K step ahead
// through two LDS stages, no register staging. A wavefront's load fills 1 KiB
// of LDS contiguously, so tiles are not padded: chunk kq of a row (BK / 8
// chunks of 16 bytes) is placed at slot row * (BK / 8) + (kq ^ swz(row)),
// which keeps the 16-byte fragment reads conflict-free.
template <int BM_, int BN_, int WM_, int WN_, int S_, int OCC_, int GM_ = 1, int BK_ = 32>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, S = S_, OCC = OCC_, GM = GM_;
    static constexpr int kCpr = BK / 8;                // 16-byte chunks per row
    static_assert(kCpr == 4 || kCpr == 8, "K steps of 32 or 64");
    static constexpr int kThreads = 64 * WM * WN;
    static constexpr int MI = BM / (32 * WM);
    static constexpr int NI = BN / (32 * WN);
    static constexpr int kAElems = BM * BK;            // no padding
    static constexpr int kWElems = BN * BK;
    static constexpr int kStageElems = kAElems + 2 * kWElems;
    static constexpr int kLdo = BN + 8;
    static constexpr int kAChunks = BM * BK / 8 / kThreads;
    static constexpr int kWChunks = BN * BK / 8 / kThreads;
    static constexpr int kLdsElems = S * kStageElems > BM * kLdo ? S * kStageElems : BM * kLdo;
    static_assert(MI >= 1 && NI >= 1 && BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "whole MFMA tiles");
    static_assert(kAChunks >= 1 && kWChunks >= 1 && BM * BK % (8 * kThreads) == 0 && BN * BK % (8 * kThreads) == 0,
                  "whole 16-byte chunks per thread");
    static_assert(S == 2, "two LDS stages");
    static_assert(BM * BN % (8 * kThreads) == 0, "whole output chunks per thread");
};

// The configurations the library launches (see the kernel-shape notes at the
// top). They differ only in the tile group: 4 row tiles for the gate_up GEMM
// (16 column tiles at inter 2048), 32 for the down projection (28 column
// tiles at hidden 7168), each the best of a sweep (gate_up: 2-4 row tiles
// 1107 TFLOP/s, 1 1094, 16 1079; down: 32 1023, 4 1011, 14 999, 7 968).
using ProdGateUp = Cfg<256, 128, 4, 2, 2, 2, 4, 64>;
using ProdDown = Cfg<256, 128, 4, 2, 2, 2, 32, 64>;

// Swizzle of a row's chunks: any 8 consecutive rows, and any 16 consecutive
// rows taken 4 or 8 apart, put the same chunk in different 16-byte bank groups.
template <int kCpr>
__device__ __forceinline__ int swz(int row) {
    if constexpr (kCpr == 4)
        return ((row >> 1) ^ (row >> 3)) & 3;
    else
        return (row ^ (row >> 3)) & 7;
}

// Slot (in 16-byte units) of chunk kq of row `row` in a swizzled tile.
template <int kCpr>
__device__ __forceinline__ int slot_of(int row, int kq) { return row * kCpr + (kq ^ swz<kCpr>(row)); }

template <int kCpr>
__device__ __forceinline__ bf16x8 frag_swz(const uint16_t* tile, int row, int kq) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(tile + slot_of<kCpr>(row, kq) * 8));
}

// s_waitcnt vmcnt(n) lgkmcnt(0) (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt in 6:4 left unconstrained, lgkmcnt in 11:8): this wavefront's loads
// up to the last n issued have landed in LDS, and its own LDS stores are done.
template <int N>
__device__ __forceinline__ void wait_loads_but() {
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// ---- the pipelined main loop ------------------------------------------------
//
// Two LDS stages of BK = 64 (four 16-wide sub-steps). Per K step the
// wavefront runs sub-steps 0-2 with the next sub-step's fragments read while
// the current sub-step's MFMAs run; then it waits for its own loads of the
// next stage and for its last fragment reads of this stage, and the block
// meets at one barrier. After it, nobody reads this stage any more and the
// next stage is complete, so the loads of the stage after next go into this
// stage's buffer and the next stage's first fragments are read, both while
// sub-step 3's MFMAs run. Only the next stage's loads are in flight at the
// barrier, so the wait is simply for all of them.
//
// Loads are issued without row bounds branches: a lane whose row lies past the
// tile's valid rows loads the last valid row instead (its results are never
// stored), so no load leaves the tensors, and the pointers are formed once per
// tile. Only a K step that crosses the end of K takes the other path, which
// writes zeros to LDS for the chunks past it (k_dim is a multiple of 8, so a
// chunk is wholly in or out).
template <class C>
struct PipeLoads {
    static constexpr int kA = C::kAChunks, kW = C::kWChunks;
    const uint16_t* pa[kA];
    const uint16_t* pg[kW];
    const uint16_t* pu[kW];
    int oa[kA], ow[kW];  // wave-uniform LDS slot of the chunk's first lane (in 16-byte units)
    int ka[kA], kw[kW];  // the lane's K offset within the step (elements)

    __device__ __forceinline__ PipeLoads(const uint16_t* a_tile, const uint16_t* g_tile, const uint16_t* u_tile,
                                         int arows, int grows, int urows, int64_t ld) {
        const int lane = static_cast<int>(threadIdx.x) % 64;
        const int wave = static_cast<int>(threadIdx.x) / 64;
#pragma unroll
        for (int i = 0; i < kA; ++i) {
            const int slot0 = i * C::kThreads + wave * 64;
            const int row = (slot0 + lane) / C::kCpr;
            const int kq = ((slot0 + lane) % C::kCpr) ^ swz<C::kCpr>(row);
            oa[i] = slot0;
            ka[i] = kq * 8;
            pa[i] = a_tile + static_cast<int64_t>(row < arows ? row : arows - 1) * ld + kq * 8;
        }
#pragma unroll
        for (int i = 0; i < kW; ++i) {
            const int slot0 = i * C::kThreads + wave * 64;
            const int row = (slot0 + lane) / C::kCpr;
            const int kq = ((slot0 + lane) % C::kCpr) ^ swz<C::kCpr>(row);
            ow[i] = slot0;
            kw[i] = kq * 8;
            pg[i] = g_tile + static_cast<int64_t>(row < grows ? row : grows - 1) * ld + kq * 8;
            pu[i] = u_tile + static_cast<int64_t>(row < urows ? row : urows - 1) * ld + kq * 8;
        }
    }

    __device__ __forceinline__ static void load(const uint16_t* src, uint16_t* dst) {
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    }

    // The same loads in buffer form (buffer_load_dwordx4 ... lds): the tile's
    // base in a scalar resource and each chunk's byte offset in one 32-bit
    // register, so a full K step needs no 64-bit address arithmetic and fewer
    // registers. Valid while every offset stays below 2^31 (kBufMaxK).
    struct Buf {
        __amdgpu_buffer_rsrc_t ra, rg, ru;
        uint32_t va[kA], vg[kW], vu[kW];
    };
    __device__ __forceinline__ Buf buffers(const uint16_t* a_tile, const uint16_t* g_tile,
                                           const uint16_t* u_tile) const {
        // dword 3 of the resource: 32-bit data format, no swizzle, as gfx9 buffer loads expect
        constexpr int kFlags = 0x00020000;
        Buf b;
        b.ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a_tile), 0, 0x7FFFFFFF, kFlags);
        b.rg = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(g_tile), 0, 0x7FFFFFFF, kFlags);
        b.ru = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(u_tile), 0, 0x7FFFFFFF, kFlags);
#pragma unroll
        for (int i = 0; i < kA; ++i) b.va[i] = static_cast<uint32_t>((pa[i] - a_tile) * 2);
#pragma unroll
        for (int i = 0; i < kW; ++i) {
            b.vg[i] = static_cast<uint32_t>((pg[i] - g_tile) * 2);
            b.vu[i] = static_cast<uint32_t>((pu[i] - u_tile) * 2);
        }
        return b;
    }
    // Load number i (A chunks first, then gate/up pairs) of full K step kt into stage st.
    __device__ __forceinline__ void issue_one(const Buf& b, uint16_t* st, int64_t kt, int i) const {
        const int soff = static_cast<int>(kt * C::BK * 2);
        auto bl = [&](__amdgpu_buffer_rsrc_t r, uint32_t voff, uint16_t* dst) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff,
                                                     0, 0);
        };
        if (i < kA) {
            bl(b.ra, b.va[i], st + oa[i] * 8);
        } else {
            const int j = (i - kA) / 2;
            if ((i - kA) % 2 == 0)
                bl(b.rg, b.vg[j], st + C::kAElems + ow[j] * 8);
            else
                bl(b.ru, b.vu[j], st + C::kAElems + C::kWElems + ow[j] * 8);
        }
    }
    __device__ __forceinline__ static void zero(uint16_t* dst) {
        *reinterpret_cast<u32x4*>(dst) = u32x4{0u, 0u, 0u, 0u};
    }

    // Loads of K step kt into `st` (one stage of LDS).
    __device__ __forceinline__ void issue(uint16_t* st, int64_t kt, int64_t k_dim) const {
        const int lane = static_cast<int>(threadIdx.x) % 64;
        const int64_t k0 = kt * C::BK;
        uint16_t* sa = st;
        uint16_t* sg = st + C::kAElems;
        uint16_t* su = st + C::kAElems + C::kWElems;
        if (k0 + C::BK <= k_dim) {
#pragma unroll
            for (int i = 0; i < kA; ++i) load(pa[i] + k0, sa + oa[i] * 8);
#pragma unroll
            for (int i = 0; i < kW; ++i) {
                load(pg[i] + k0, sg + ow[i] * 8);
                load(pu[i] + k0, su + ow[i] * 8);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kA; ++i) {
                if (k0 + ka[i] < k_dim)
                    load(pa[i] + k0, sa + oa[i] * 8);
                else
                    zero(sa + (oa[i] + lane) * 8);
            }
#pragma unroll
            for (int i = 0; i < kW; ++i) {
                if (k0 + kw[i] < k_dim) {
                    load(pg[i] + k0, sg + ow[i] * 8);
                    load(pu[i] + k0, su + ow[i] * 8);
                } else {
                    zero(sg + (ow[i] + lane) * 8);
                    zero(su + (ow[i] + lane) * 8);
                }
            }
        }
    }
};

template <class C, bool kBuf>
__device__ __forceinline__ void mainloop_pipe(uint16_t* lds, const uint16_t* a_tile, const uint16_t* g_tile,
                                              const uint16_t* u_tile, int arows, int grows, int urows,
                                              int64_t k_dim, f32x16 (&acc_g)[C::MI][C::NI],
                                              f32x16 (&acc_u)[C::MI][C::NI]) {
    constexpr int MI = C::MI, NI = C::NI, KK = C::BK / 16;
    static_assert(C::S == 2 && KK >= 2, "two stages of at least two sub-steps");
    const int lane = static_cast<int>(threadIdx.x) % 64;
    const int wave = static_cast<int>(threadIdx.x) / 64;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const PipeLoads<C> ld(a_tile, g_tile, u_tile, arows, grows, urows, k_dim);
    const int64_t nk = (k_dim + C::BK - 1) / C::BK;

    bf16x8 fa[2][MI], fg[2][NI], fu[2][NI];
    auto read = [&](const uint16_t* stage, int b, int kk) {
        const uint16_t* sa = stage;
        const uint16_t* sg = stage + C::kAElems;
        const uint16_t* su = stage + C::kAElems + C::kWElems;
        const int kq = kk * 2 + lane / 32;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
            fa[b][mi] = frag_swz<C::kCpr>(sa, wm * (C::BM / C::WM) + mi * 32 + lane % 32, kq);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
            fg[b][ni] = frag_swz<C::kCpr>(sg, wn * (C::BN / C::WN) + ni * 32 + lane % 32, kq);
            fu[b][ni] = frag_swz<C::kCpr>(su, wn * (C::BN / C::WN) + ni * 32 + lane % 32, kq);
        }
    };
    auto mfma = [&](int b) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                acc_g[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[b][mi], fg[b][ni], acc_g[mi][ni], 0, 0, 0);
                acc_u[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[b][mi], fu[b][ni], acc_u[mi][ni], 0, 0, 0);
            }
    };
    // one fragment read of the next sub-step after each of this sub-step's
    // first MFMAs (left to itself, the compiler issued the reads after the
    // MFMAs and waited for them at the start of every sub-step)
    auto interleave = [&]() {
        constexpr int kReads = MI + 2 * NI, kMfmas = 2 * MI * NI;
#pragma unroll
        for (int i = 0; i < kReads; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kMfmas - kReads, 0);
    };

    ld.issue(lds, 0, k_dim);
    wait_loads_but<0>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (nk > 1) ld.issue(lds + C::kStageElems, 1, k_dim);
    read(lds, 0, 0);

    int64_t kt = 0;
    if constexpr (kBuf) {
        // While the step after next is a full K step, the last sub-step issues
        // its loads in buffer form one after each MFMA, with the next step's
        // first fragment reads in between, in a branch-free loop body. Issued
        // together before the MFMAs, the loads held the wavefronts at issue
        // while the MFMA units idled (1072 against 1174 TFLOP/s for gate_up).
        constexpr int kLoads = C::kAChunks + 2 * C::kWChunks, kReads = MI + 2 * NI, kMf = 2 * MI * NI;
        static_assert(kLoads <= kMf && kReads <= kMf, "one load and one read per MFMA at most");
        const typename PipeLoads<C>::Buf bufs = ld.buffers(a_tile, g_tile, u_tile);
        const int64_t nmain = nk - (k_dim % C::BK == 0 ? 2 : 3);
        constexpr int b = (KK - 1) & 1;
        for (; kt < nmain; ++kt) {
            uint16_t* cur = lds + (kt & 1) * C::kStageElems;
            const uint16_t* nxt = lds + ((kt + 1) & 1) * C::kStageElems;
#pragma unroll
            for (int kk = 0; kk + 1 < KK; ++kk) {
                read(cur, (kk + 1) & 1, kk + 1);
                mfma(kk & 1);
                interleave();
                __builtin_amdgcn_sched_barrier(0);
            }
            wait_loads_but<0>();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            const int kq = lane / 32;
#pragma unroll
            for (int i = 0; i < kMf; ++i) {
                const int mi = i / (2 * NI), ni = (i / 2) % NI;
                if (i % 2 == 0)
                    acc_g[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[b][mi], fg[b][ni], acc_g[mi][ni], 0, 0, 0);
                else
                    acc_u[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[b][mi], fu[b][ni], acc_u[mi][ni], 0, 0, 0);
                if (i < kLoads) ld.issue_one(bufs, cur, kt + 2, i);
                if (i < MI) {
                    fa[0][i] = frag_swz<C::kCpr>(nxt, wm * (C::BM / C::WM) + i * 32 + lane % 32, kq);
                } else if (i < kReads) {
                    const int j = (i - MI) / 2;
                    const uint16_t* w = nxt + C::kAElems + ((i - MI) % 2) * C::kWElems;
                    const bf16x8 f = frag_swz<C::kCpr>(w, wn * (C::BN / C::WN) + j * 32 + lane % 32, kq);
                    if ((i - MI) % 2 == 0)
                        fg[0][j] = f;
                    else
                        fu[0][j] = f;
                }
                __builtin_amdgcn_sched_barrier(0);  // keep this order: MFMA, load, read
            }
        }
    }
    for (; kt < nk; ++kt) {
        uint16_t* cur = lds + (kt & 1) * C::kStageElems;
        uint16_t* nxt = lds + ((kt + 1) & 1) * C::kStageElems;
#pragma unroll
        for (int kk = 0; kk + 1 < KK; ++kk) {
            read(cur, (kk + 1) & 1, kk + 1);
            mfma(kk & 1);
            interleave();
            __builtin_amdgcn_sched_barrier(0);
        }
        if (kt + 1 < nk) {
            // own loads of the next stage landed, own reads of this stage done; then the block meets
            wait_loads_but<0>();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            if (kt + 2 < nk) ld.issue(cur, kt + 2, k_dim);
            read(nxt, 0, 0);
        }
        mfma((KK - 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Epilogues: the clamped SwiGLU of (gate, up) (two weight tensors, the same
// columns of each), or the router-weight multiply of a single weight tensor's
// output (the block's two weight tiles are then consecutive column ranges of
// it), stored as bf16 or fp32.
enum class Epi { kSwiglu, kRouterBf16, kRouterF32 };

// A grouped GEMM over rows grouped by expert: the reduction runs over k_dim
// (hidden for gate_up, inter for the down projection); n_dim is the width of
// each weight tensor's output (inter for gate_up, hidden for down).
template <class C, Epi kEpi, bool kWriteX, bool kBuf>
__global__ __launch_bounds__(C::kThreads) __attribute__((amdgpu_waves_per_eu(C::OCC))) void grouped_gemm_kernel(
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ w1, const uint16_t* __restrict__ w2,
    const int32_t* __restrict__ offs, const float* __restrict__ probs, void* __restrict__ out,
    uint16_t* __restrict__ x_out, int64_t tokens, int64_t k_dim, int64_t n_dim, int64_t experts, float L,
    int64_t n_tiles, int64_t n_blocks) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[C::kLdsElems];
    constexpr int MI = C::MI, NI = C::NI;
    constexpr bool kRouter = kEpi != Epi::kSwiglu;

    const int64_t logical = blockIdx.x;
    if (logical >= n_blocks) return;
    int64_t mt, nt;
    tile_of(logical, n_blocks / n_tiles, n_tiles, C::GM, &mt, &nt);
    const TileRows tr = find_row_tile(offs, tokens, experts, mt, C::BM);
    if (tr.rows == 0) return;
    // first output column of each weight tile (gate and up: the same columns;
    // router: two consecutive ranges of one weight tensor) and its valid width
    const int64_t col1 = nt * (kRouter ? 2 * C::BN : C::BN);
    const int64_t col2 = kRouter ? col1 + C::BN : col1;
    const int ncols1 = static_cast<int>(n_dim - col1 < C::BN ? n_dim - col1 : C::BN);
    const int ncols2 = static_cast<int>(n_dim - col2 <= 0 ? 0 : (n_dim - col2 < C::BN ? n_dim - col2 : C::BN));

    const uint16_t* a_tile = a + tr.row0 * k_dim;
    const uint16_t* g_tile = w1 + (tr.expert * n_dim + col1) * k_dim;
    // with no second tile (ncols2 == 0) its loads repeat the first tile's rows and go unused
    const uint16_t* u_tile = w2 + (tr.expert * n_dim + (ncols2 > 0 ? col2 : col1)) * k_dim;

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

    mainloop_pipe<C, kBuf>(lds, a_tile, g_tile, u_tile, tr.rows, ncols1, ncols2 > 0 ? ncols2 : 1, k_dim, acc_g, acc_u);
    __syncthreads();  // all fragment reads done before the buffers become the staging tile

    uint16_t* stage = lds;
    if constexpr (kEpi == Epi::kSwiglu) {
        uint16_t* y = static_cast<uint16_t*>(out);
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
        store_tile<C>(stage, y, n_dim, tr.row0, tr.rows, col1, n_dim);
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
            store_tile<C>(stage, x_out, 2 * n_dim, tr.row0, tr.rows, col1, n_dim);
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
            store_tile<C>(stage, x_out + n_dim, 2 * n_dim, tr.row0, tr.rows, col1, n_dim);
        }
    } else if constexpr (kEpi == Epi::kRouterF32) {
        // fp32 staged through LDS, one weight tile (BM x BN floats, all of the
        // LDS) at a time, then stored as 16-byte row-contiguous chunks. The
        // column is XOR-swizzled by bit 2 of the row, so the two halves of a
        // wavefront's write (rows r and r + 4) fall in different banks. Stores
        // straight from the accumulators (4 bytes per lane) ran 13% slower.
        static_assert(C::BM * C::BN * 4 <= C::kLdsElems * 2, "an fp32 tile fits the LDS");
        float* o = static_cast<float*>(out);
        float* stf = reinterpret_cast<float*>(lds);
        auto sw = [](int r, int c) { return c ^ (((r >> 2) & 1) * 32); };
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int ncols = half == 0 ? ncols1 : ncols2;
            const int64_t colb = half == 0 ? col1 : col2;
            if (ncols == 0) break;
            if (half == 1) __syncthreads();  // the first half's stores have read the staging tile
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int r = acc_row<C>(wm, mi, j, lane);
                    const float p = r < tr.rows ? probs[tr.row0 + r] : 0.0f;
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni) {
                        const float v = half == 0 ? acc_g[mi][ni][j] : acc_u[mi][ni][j];
                        stf[r * C::BN + sw(r, acc_col<C>(wn, ni, lane))] = round_bf16(v) * p;
                    }
                }
            __syncthreads();
            constexpr int kChunks = C::BM * C::BN / 4 / C::kThreads;
#pragma unroll
            for (int i = 0; i < kChunks; ++i) {
                const int c = static_cast<int>(threadIdx.x) + i * C::kThreads;
                const int row = c / (C::BN / 4), cq = c % (C::BN / 4);
                if (row < tr.rows && cq * 4 < ncols)
                    store_nt16(o + (tr.row0 + row) * n_dim + colb + cq * 4,
                               *reinterpret_cast<const u32x4*>(stf + row * C::BN + sw(row, cq * 4)));
            }
        }
    } else {
        uint16_t* o = static_cast<uint16_t*>(out);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            if (half == 1) __syncthreads();  // the first half's stores have read the staging tile
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int r = acc_row<C>(wm, mi, j, lane);
                    const float p = r < tr.rows ? probs[tr.row0 + r] : 0.0f;
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni) {
                        const float v = half == 0 ? acc_g[mi][ni][j] : acc_u[mi][ni][j];
                        stage[r * C::kLdo + acc_col<C>(wn, ni, lane)] = to_bf16(round_bf16(v) * p);
                    }
                }
            __syncthreads();
            if (half == 0)
                store_tile<C>(stage, o, n_dim, tr.row0, tr.rows, col1, col1 + ncols1);
            else if (ncols2 > 0)
                store_tile<C>(stage, o, n_dim, tr.row0, tr.rows, col2, col2 + ncols2);
        }
    }
}

// Largest reduction length for the buffer-form loads: every byte offset from a
// tile's base, (BM - 1) rows plus a whole row of k_dim bf16 values, stays
// below 2^31.
template <class C>
constexpr int64_t kBufMaxK = ((int64_t{1} << 31) - 1) / (2 * (C::BM + 1));

template <class C, Epi kEpi, bool kWriteX>
void launch_kernel(bool buf, int64_t grid, hipStream_t st, const uint16_t* a, const uint16_t* w1, const uint16_t* w2,
                   const int32_t* offs, const float* probs, void* out, uint16_t* x_out, int64_t tokens, int64_t k_dim,
                   int64_t n_dim, int64_t experts, float limit, int64_t n_tiles, int64_t n_blocks) {
    if (buf)
        hipLaunchKernelGGL((grouped_gemm_kernel<C, kEpi, kWriteX, true>), dim3(static_cast<unsigned>(grid)),
                           dim3(C::kThreads), 0, st, a, w1, w2, offs, probs, out, x_out, tokens, k_dim, n_dim, experts,
                           limit, n_tiles, n_blocks);
    else
        hipLaunchKernelGGL((grouped_gemm_kernel<C, kEpi, kWriteX, false>), dim3(static_cast<unsigned>(grid)),
                           dim3(C::kThreads), 0, st, a, w1, w2, offs, probs, out, x_out, tokens, k_dim, n_dim, experts,
                           limit, n_tiles, n_blocks);
}

template <class C, Epi kEpi>
int launch_grouped(const uint16_t* a, const uint16_t* w1, const uint16_t* w2, const int32_t* offs,
                   const float* probs, void* out, uint16_t* x_out, int64_t tokens, int64_t k_dim, int64_t n_dim,
                   int64_t experts, float limit, hipStream_t st) {
    int64_t n_tiles, n_blocks;
    const int64_t grid = grouped_grid(tokens, n_dim, kEpi == Epi::kSwiglu ? C::BN : 2 * C::BN, experts, C::BM, &n_tiles,
                                         &n_blocks);
    if (grid == 0) return MOE_EPI_ERR_BAD_SHAPE;
    const bool buf = k_dim <= kBufMaxK<C>;
    (void)hipGetLastError();
    if (kEpi == Epi::kSwiglu && x_out)
        launch_kernel<C, kEpi, true>(buf, grid, st, a, w1, w2, offs, probs, out, x_out, tokens, k_dim, n_dim, experts,
                                     limit, n_tiles, n_blocks);
    else
        launch_kernel<C, kEpi, false>(buf, grid, st, a, w1, w2, offs, probs, out, x_out, tokens, k_dim, n_dim, experts,
                                      limit, n_tiles, n_blocks);
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
    return launch_grouped<ProdGateUp, Epi::kSwiglu>(a, w_gate, w_up, offs, probs, y, x_out, tokens, hidden, inter, experts,
                                              limit, as_stream(stream));
}

extern "C" int grouped_down_router_fwd(const uint16_t* h, const uint16_t* w_down, const int32_t* offs,
                                       const float* probs, void* out, int out_dtype, int64_t tokens, int64_t inter,
                                       int64_t hidden, int64_t experts, void* stream) {
    if (out_dtype != MOE_EPI_BF16 && out_dtype != MOE_EPI_F32) return MOE_EPI_ERR_BAD_DTYPE;
    if (tokens < 0 || tokens > INT32_MAX || inter <= 0 || hidden <= 0 || experts <= 0 || inter % 8 != 0 ||
        hidden % 8 != 0)
        return MOE_EPI_ERR_BAD_SHAPE;
    if (experts > INT64_MAX / 4 / hidden)  // before experts * hidden is formed
        return MOE_EPI_ERR_BAD_SHAPE;
    const int eo = elem_bytes(out_dtype);
    int64_t hb, wb, ob, pb, fb;
    if (!bytes_ok(tokens, inter, 2, &hb) || !bytes_ok(experts * hidden, inter, 2, &wb) ||
        !bytes_ok(tokens, hidden, eo, &ob) || !bytes_ok(tokens, 1, 4, &pb) || !bytes_ok(experts, 1, 4, &fb))
        return MOE_EPI_ERR_BAD_SHAPE;
    if (tokens == 0) return MOE_EPI_SUCCESS;
    if (!h || !w_down || !offs || !probs || !out) return MOE_EPI_ERR_NULL_POINTER;
    if (!aligned(h, 16) || !aligned(w_down, 16) || !aligned(out, 16) || !aligned(offs, 4) || !aligned(probs, 4))
        return MOE_EPI_ERR_MISALIGNED;
    const Range ro = range_of(out, ob);
    if (overlaps(ro, range_of(h, hb)) || overlaps(ro, range_of(w_down, wb)) || overlaps(ro, range_of(offs, fb)) ||
        overlaps(ro, range_of(probs, pb)))
        return MOE_EPI_ERR_ALIAS;
    if (out_dtype == MOE_EPI_F32)
        return launch_grouped<ProdDown, Epi::kRouterF32>(h, w_down, w_down, offs, probs, out, nullptr, tokens, inter,
                                                     hidden, experts, 1.0f, as_stream(stream));
    return launch_grouped<ProdDown, Epi::kRouterBf16>(h, w_down, w_down, offs, probs, out, nullptr, tokens, inter, hidden,
                                                  experts, 1.0f, as_stream(stream));
}
