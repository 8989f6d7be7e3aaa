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
//     eight wavefronts (4 x 2) of 64 x 64 each: 4 x 4 v_mfma_f32_16x16x32_bf16
//     tiles for gate and 4 x 4 for up, 128 fp32 accumulators per lane, two
//     wavefronts per SIMD, one block per CU (128 KiB of LDS).
//   * The MFMA shape: under sustained MFMA load this part is power-limited,
//     and the 16 x 16 x 32 instruction draws less power per FLOP than the
//     32 x 32 x 16 one. A loop of nothing but MFMAs on all CUs, two wavefronts
//     per SIMD, held 2.0 GHz and 2020-2055 TFLOP/s with the first against
//     1.75 GHz and 1777-1790 TFLOP/s with the second (both at about 97% of the
//     rate their clock allows).
//   * Operands go from global memory straight into LDS (buffer_load_dwordx4
//     ... lds), K steps of 64, two LDS stages: the next step's loads are in
//     flight while this step's MFMAs run, with no registers spent on staging.
//     Tiles are not padded (a wavefront's load fills 1 KiB contiguously); an
//     XOR swizzle of each row's 16-byte chunks keeps the fragment reads
//     conflict-free.
//   * A K step is two 32-wide sub-steps of 32 MFMAs each. The next sub-step's
//     fragments are read from LDS while the current one's MFMAs run, each
//     fragment register refilled right after the last MFMA that uses it. One
//     barrier per K step, between its sub-steps, a bare s_barrier after
//     explicit waits (a __syncthreads() fence would also wait for the loads
//     still in flight); the loads of the step after next and the next step's
//     first fragments are issued while the second sub-step's MFMAs run, the
//     loads by one wavefront per SIMD, one after every second MFMA (the other
//     wavefront on the SIMD then never waits at a load's issue); the wave
//     index is made uniform, so each load's LDS address (M0) is formed in
//     scalar registers. The loop runs from one barrier to
//     the next, so that the compiler counts the fragment reads in flight
//     instead of waiting for all of them at the top of every K step.
//   * Tiles never straddle experts: each block finds its expert and row range
//     from offs on the device (no host copy of offs), so a grid sized for
//     the worst case, ceil(tokens / 256) + experts row tiles, covers any split.
//   * Tile order: tiles are visited in groups of row tiles (2 for gate_up, 32
//     for the down projection), the row tile changing fastest, so that the
//     blocks running together on one XCD share both their A tiles and their
//     weight tiles in that XCD's L2. The hardware hands consecutive block ids
//     to the 8 XCDs in turn, and the kernel keeps that placement: all XCDs
//     then work on neighbouring tiles of the same expert, and their L2 misses
//     on its weights and activations hit the shared Infinity Cache. Giving
//     each XCD a contiguous range of tiles instead puts the XCDs on different
//     experts: gate_up 1061 TFLOP/s against 1107, the down projection 1008
//     against 1023.
//   * Epilogue: accumulators are rounded to bf16 (two per conversion), the
//     SwiGLU or the router multiply is applied, and each output tile is staged
//     through LDS so that global stores are 16-byte, row-contiguous accesses.
//     The MFMAs take the weight fragment first, so a lane's accumulators hold
//     four consecutive columns of one row; one v_permlane16_swap per pair of
//     tiles gives each lane eight consecutive bf16 columns, written to LDS
//     with one 16-byte write.
// Measured at 131072 x 7168 x 2048 with 8 experts, A/B in one process on one
// box: with 32 x 32 x 16 MFMAs (the loop above in its earlier form, four
// 16-wide sub-steps per K step) down 3.309 ms and gate_up 6.309 ms; with
// 16 x 16 x 32 MFMAs 3.210 and 6.109; with the loop from barrier to barrier
// 3.121 and 6.019 (1233 and 1279 TFLOP/s); with M0 from scalar registers 3.04
// and 5.86 ms on another box; with one loading wavefront per SIMD 0.2-1.5%
// faster again (three boxes). Timing-only copies of the earlier
// loop (TFLOP/s, gate_up / down): MFMAs and epilogue alone 1899 / 1698, plus
// the barrier 1885 / 1687, plus the fragment reads 1684 / 1532, plus the loads
// instead of the reads 1374 / 1312: the loads set the pace. Variants that did
// not help: the A fragments of two sub-steps held, so that they are read a
// sub-step ahead (no change), all eight wavefronts loading one after every
// second MFMA (4% slower on gate_up), half of the loads moved into the next
// sub-step (4-6% slower), two loading wavefronts (4% slower), groups of 4
// and 16 row tiles (1% slower), each XCD given a contiguous range of tiles
// (7-20% slower). Earlier, with the
// 32 x 32 x 16 loop: register-staged loads with padded LDS ran at 746-918
// TFLOP/s over 22 tile shapes; K steps of 32 with 3-5 stages (850-912), two
// 128 x 128 blocks per CU (870-890), an L2 prefetch two to four steps ahead
// (930), A tiles three stages deep (929-962), four wavefronts of 128-row
// tiles (950-1144), raised wave priority around the MFMAs (997), a ping-pong
// of two wavefront groups (885-925) and accumulators in AGPRs (no change) did
// not help either.
#include "epi_common.h"
#include "grouped_map.h"
#include "swiglu_math.h"

namespace moe_epi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Accumulator layout. v_mfma_f32_16x16x32_bf16 leaves C[4*(l/16) + j][l%16] in
// register j of lane l. The MFMAs take the weight fragment as their first
// operand, so that C's rows run along the output columns: lane l of tile
// (mi, ni) holds the outputs of block-tile row acc_row(mi) and of the four
// consecutive columns from acc_col(ni), one per register.
template <class C>
__device__ __forceinline__ int acc_row(int wm, int mi, int lane) {
    return wm * (C::BM / C::WM) + mi * 16 + lane % 16;
}
template <class C>
__device__ __forceinline__ int acc_col(int wn, int ni, int lane) {
    return wn * (C::BN / C::WN) + ni * 16 + 4 * (lane / 16);
}

// Two fp32 values rounded to bf16 and packed, the first in the low half (one
// two-source v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// Two fp32 values rounded to bf16 and widened back (one conversion for both).
__device__ __forceinline__ f32x2 round2_bf16(float a, float b) {
    const uint32_t w = pk_bf16(a, b);
    return f32x2{__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u)};
}

// Eight consecutive bf16 outputs of one row from two tiles of the same rows,
// pair(t, j) giving the outputs of registers j and j + 1 (j = 0 or 2) of tile
// t (0 or 1). Before the exchange lane l holds columns 4g .. 4g + 3 of both
// tiles (g = l / 16, the lane's group of 16); v_permlane16_swap trades the
// second tile's values of groups 0 and 2 for the first tile's values of
// groups 1 and 3, after which a lane of group g holds columns
// 8 (g / 2) .. 8 (g / 2) + 7 of tile g % 2 in order, one 16-byte chunk.
template <class F>
__device__ __forceinline__ u32x4 row_chunk(F&& pair) {
    auto pk = [&](int t, int j) {
        const f32x2 v = pair(t, j);
        return pk_bf16(v[0], v[1]);
    };
    const uint32_t x0 = pk(0, 0), x1 = pk(0, 2), y0 = pk(1, 0), y1 = pk(1, 2);
    const auto s0 = __builtin_amdgcn_permlane16_swap(x0, y0, false, false);
    const auto s1 = __builtin_amdgcn_permlane16_swap(x1, y1, false, false);
    return u32x4{s0[0], s1[0], s0[1], s1[1]};
}
// The tile (0 or 1) of the lane's chunk and its first column within that tile.
__device__ __forceinline__ int chunk_tile(int lane) { return (lane / 16) % 2; }
__device__ __forceinline__ int chunk_col(int lane) { return 8 * (lane / 32); }

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
template <int BM_, int BN_, int WM_, int WN_, int S_, int OCC_, int GM_ = 1, int BK_ = 64>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, S = S_, OCC = OCC_, GM = GM_;
    static constexpr int kCpr = BK / 8;                // 16-byte chunks per row
    static_assert(kCpr == 8, "K steps of 64: two 32-wide MFMA sub-steps");
    static constexpr int kThreads = 64 * WM * WN;
    static constexpr int MI = BM / (16 * WM);           // 16 x 16 MFMA tiles per wavefront
    static constexpr int NI = BN / (16 * WN);
    static constexpr int kAElems = BM * BK;            // no padding
    static constexpr int kWElems = BN * BK;
    static constexpr int kStageElems = kAElems + 2 * kWElems;
    static constexpr int kLdo = BN + 8;
    // The global -> LDS loads are issued by four of the eight wavefronts (one
    // per SIMD), so that the other wavefront on each SIMD never waits at a
    // load's issue and keeps the MFMA unit fed: 0.2-1.5% faster than all eight
    // loading (three boxes), two loading wavefronts 4% slower.
    static constexpr int kLoadWaves = 4, kLoadThreads = 64 * kLoadWaves;
    static constexpr int kAChunks = BM * BK / 8 / kLoadThreads;
    static constexpr int kWChunks = BN * BK / 8 / kLoadThreads;
    static constexpr int kLdsElems = S * kStageElems > BM * kLdo ? S * kStageElems : BM * kLdo;
    static_assert(MI >= 1 && NI >= 2 && NI % 2 == 0 && BM % (16 * WM) == 0 && BN % (16 * WN) == 0,
                  "whole MFMA tiles, pairs of column tiles for the epilogue's exchange");
    static_assert(kAChunks >= 1 && kWChunks >= 1 && BM * BK % (8 * kLoadThreads) == 0 && BN * BK % (8 * kLoadThreads) == 0,
                  "whole 16-byte chunks per thread");
    static_assert(S == 2, "two LDS stages");
    static_assert(BM * BN % (8 * kThreads) == 0, "whole output chunks per thread");
};

// The configurations the library launches (see the kernel-shape notes at the
// top). They differ only in the tile group: 2 row tiles for the gate_up GEMM
// (16 column tiles at inter 2048), 32 for the down projection (28 column
// tiles at hidden 7168), each the best of a sweep. With the 16 x 16 x 32 loop,
// A/B in one process: gate_up 2 row tiles 5.99 ms against 6.05 for 4; down
// 32 3.11 ms against 3.13 for 16. With the 32 x 32 x 16 loop: gate_up 2 row
// tiles 6.27-6.34 ms, 4 6.31-6.41, 1 6.40, 3 6.69, 8 6.49; down 32
// 3.29-3.30 ms, 16 3.31-3.32, 24 3.33, 48 3.34, 64 3.35.
using ProdGateUp = Cfg<256, 128, 4, 2, 2, 2, 2, 64>;
using ProdDown = Cfg<256, 128, 4, 2, 2, 2, 32, 64>;

// Swizzle of a row's eight chunks. A fragment read takes one chunk of 16
// consecutive rows starting at a multiple of 16; with rows of 128 bytes, row t
// of those puts it in 16-byte bank group (t % 2) * 8 + (kq ^ swz), and over the
// 16 rows these are the 16 different groups of the 64 banks (any 8 of the rows
// from a multiple of 8: 8 different groups of 32 banks). It depends on the row
// modulo 16 only, so the fragments of tiles 16 rows apart sit at a constant
// distance and share their address register.
template <int kCpr>
__device__ __forceinline__ int swz(int row) {
    static_assert(kCpr == 8, "rows of eight chunks");
    return (row & 7) ^ ((row >> 3) & 1);
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

// A block barrier for LDS hazards only: this wavefront's LDS reads and writes
// are complete, then the block meets. __syncthreads() would also wait for every
// global store still in flight (its release fence), which in the epilogue put
// the full store latency between one staged output tile and the next.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt left free (gfx9 encoding)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---- the pipelined main loop ------------------------------------------------
//
// Two LDS stages of BK = 64, each two 32-wide sub-steps of
// v_mfma_f32_16x16x32_bf16. Per K step the wavefront runs sub-step 0 with
// sub-step 1's fragments read while its MFMAs run; then it waits for its own
// loads of the next stage and for its fragment reads of this stage, and the
// block meets at one barrier. After it, nobody reads this stage any more and
// the next stage is complete, so the loads of the stage after next go into
// this stage's buffer and the next stage's first fragments are read, both
// while sub-step 1's MFMAs run. Only the next stage's loads are in flight at
// the barrier, so the wait is simply for all of them.
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
        // wave-uniform, so that each load's LDS address (M0) is formed in scalar
        // registers: gate_up 5.86 against 5.97 ms, down 3.04 against 3.07 ms
        const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / 64);
#pragma unroll
        for (int i = 0; i < kA; ++i) {
            const int slot0 = i * C::kLoadThreads + (wave % C::kLoadWaves) * 64;
            const int row = (slot0 + lane) / C::kCpr;
            const int kq = ((slot0 + lane) % C::kCpr) ^ swz<C::kCpr>(row);
            oa[i] = slot0;
            ka[i] = kq * 8;
            pa[i] = a_tile + static_cast<int64_t>(row < arows ? row : arows - 1) * ld + kq * 8;
        }
#pragma unroll
        for (int i = 0; i < kW; ++i) {
            const int slot0 = i * C::kLoadThreads + (wave % C::kLoadWaves) * 64;
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
    // Load number i (numbered as in issue_one) of the K step kt that crosses
    // the end of K, in pointer form from the buffer offsets: chunks past k_dim
    // are written as zeros.
    __device__ __forceinline__ void issue_one_tail(const Buf& b, const uint16_t* a_tile, const uint16_t* g_tile,
                                                   const uint16_t* u_tile, uint16_t* st, int64_t kt, int i,
                                                   int64_t k_dim) const {
        // the thread index through an empty asm, so that nothing derived from
        // it is hoisted out of the main loop to sit in registers for this path
        int tid = static_cast<int>(threadIdx.x);
        asm volatile("" : "+v"(tid));
        const int lane = tid % 64, wave = tid / 64;
        const uint16_t* tile;
        uint32_t voff;
        uint16_t* dst;
        int slot0;
        if (i < kA) {
            slot0 = i * C::kLoadThreads + (wave % C::kLoadWaves) * 64;
            tile = a_tile;
            voff = b.va[i];
            dst = st + slot0 * 8;
        } else {
            const int j = (i - kA) / 2;
            slot0 = j * C::kLoadThreads + (wave % C::kLoadWaves) * 64;
            const bool up = (i - kA) % 2 == 1;
            tile = up ? u_tile : g_tile;
            voff = up ? b.vu[j] : b.vg[j];
            dst = st + C::kAElems + (up ? C::kWElems : 0) + slot0 * 8;
        }
        const int row = (slot0 + lane) / C::kCpr;
        const int kq = ((slot0 + lane) % C::kCpr) ^ swz<C::kCpr>(row);
        const int64_t k0 = kt * C::BK;
        if (k0 + kq * 8 < k_dim)
            load(tile + voff / 2 + k0, dst);
        else
            zero(dst + lane * 8);
    }

    // Loads of K step kt into `st` (one stage of LDS).
    __device__ __forceinline__ void issue(uint16_t* st, int64_t kt, int64_t k_dim) const {
        if (__builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / 64) >= C::kLoadWaves) return;
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

// The main loop's three forms, chosen by the host from k_dim.
enum Loop : int {
    kPtrLoop = 0,   // pointer-form loads (k_dim above kBufMaxK)
    kBufLoop = 1,   // buffer-form loads, k_dim a multiple of BK
    kBufTail = 2,   // buffer-form loads, and a last K step that crosses the end of K
};

template <class C, int kLoop>
__device__ __forceinline__ void mainloop_pipe(uint16_t* lds, const uint16_t* a_tile, const uint16_t* g_tile,
                                              const uint16_t* u_tile, int arows, int grows, int urows,
                                              int64_t k_dim, f32x4 (&acc_g)[C::MI][C::NI],
                                              f32x4 (&acc_u)[C::MI][C::NI]) {
    constexpr int MI = C::MI, NI = C::NI, kMf = 2 * MI * NI;
    static_assert(C::S == 2 && C::BK == 64, "two stages of two 32-wide sub-steps");
    const int lane = static_cast<int>(threadIdx.x) % 64;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / 64);
    const int wm = wave / C::WN, wn = wave % C::WN;
    const PipeLoads<C> ld(a_tile, g_tile, u_tile, arows, grows, urows, k_dim);
    const int64_t nk = (k_dim + C::BK - 1) / C::BK;

    // Fragments (16 rows x 32 k, eight bf16 per lane: row lane % 16, one of
    // the sub-step's four 16-byte chunks of that row per group of 16 lanes),
    // one sub-step's worth: each is replaced by the next sub-step's once the
    // MFMAs that use it have issued, which keeps the loop within 256 registers
    // beside the 128 accumulators. Which lanes read which chunk is free as long
    // as A and the weights agree; lanes l and l + 32 read adjacent chunks (as
    // the two halves of a 32 x 32 fragment did): with lanes l and l + 16 on
    // adjacent chunks instead, the same reads kept the LDS busy 46% of the
    // time against 24%, and the kernels ran 0.7-1.3% slower.
    bf16x8 fa[MI], fg[NI], fu[NI];
    const int kq0 = ((lane / 16) & 1) * 2 + lane / 32;
    auto read_a = [&](const uint16_t* stage, int kk, int mi) {
        fa[mi] = frag_swz<C::kCpr>(stage, wm * (C::BM / C::WM) + mi * 16 + lane % 16, 4 * kk + kq0);
    };
    auto read_w = [&](const uint16_t* stage, int kk, int ni) {
        const int row = wn * (C::BN / C::WN) + ni * 16 + lane % 16;
        fg[ni] = frag_swz<C::kCpr>(stage + C::kAElems, row, 4 * kk + kq0);
        fu[ni] = frag_swz<C::kCpr>(stage + C::kAElems + C::kWElems, row, 4 * kk + kq0);
    };
    // MFMA i of a sub-step: the column tile outermost, then the row tile, gate
    // before up; weight fragment first (see acc_row / acc_col).
    auto mfma = [&](int i) {
        const int ni = i / (2 * MI), mi = (i / 2) % MI;
        if (i % 2 == 0)
            acc_g[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fg[ni], fa[mi], acc_g[mi][ni], 0, 0, 0);
        else
            acc_u[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fu[ni], fa[mi], acc_u[mi][ni], 0, 0, 0);
    };
    // The next sub-step's reads (sub-step kk of `stage`) that follow MFMA i:
    // a column tile's weight fragments after the last MFMA using them, and in
    // the last column tile, each A fragment after its last MFMA.
    auto reads_after = [&](int i, const uint16_t* stage, int kk) {
        if (i >= 2 * MI * (NI - 1) && i % 2 == 1) read_a(stage, kk, (i / 2) % MI);
        if (i % (2 * MI) == 2 * MI - 1) read_w(stage, kk, i / (2 * MI));
    };
    // A sub-step with the next one's reads, pinned in this order (left to
    // itself, the compiler issued the reads after the MFMAs and waited for
    // them at the start of every sub-step).
    auto substep = [&](const uint16_t* next_stage, int next_kk) {
#pragma unroll
        for (int i = 0; i < kMf; ++i) {
            mfma(i);
            reads_after(i, next_stage, next_kk);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto block_barrier = [&]() {  // own loads landed, own reads done, then the block meets
        wait_loads_but<0>();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    ld.issue(lds, 0, k_dim);
    block_barrier();
    if (nk > 1) ld.issue(lds + C::kStageElems, 1, k_dim);
    // the first sub-step's fragments, read in the loop's order, so that the
    // waits at the top of the loop can count the reads still in flight
#pragma unroll
    for (int i = 0; i < kMf; ++i) reads_after(i, lds, 0);

    if constexpr (kLoop != kPtrLoop) {
        // The loop runs from the middle of one K step to the middle of the
        // next, so that its head follows a barrier (where every read has been
        // waited for) and the waits between sub-steps are counted exactly.
        // Sub-step 1 of step kt issues the loads of step kt + 2 (in the loading
        // wavefronts), one after every kEvery-th MFMA, between the reads of
        // step kt + 1's first fragments: in buffer form while that step is a full K step, in
        // pointer form with zeros past K for the step that crosses the end of
        // K (uniform branches). Issued together before the MFMAs, the loads held
        // the wavefronts at issue while the MFMA units idled (1072 against 1174
        // TFLOP/s for gate_up). The step that crosses the end of K has a form of
        // its own (kBufTail): its zero fill writes LDS, after which the compiler
        // can no longer count the fragment reads in flight and waits for all of
        // them at the start of every sub-step.
        constexpr int kLoads = C::kAChunks + 2 * C::kWChunks, kEvery = kMf / kLoads;
        static_assert(kEvery >= 1, "one load per MFMA at most");
        const typename PipeLoads<C>::Buf bufs = ld.buffers(a_tile, g_tile, u_tile);
        // k_dim <= kBufMaxK here, so step counts fit 32 bits (scalar compares)
        const int nk32 = static_cast<int>(nk), nfull = static_cast<int>(k_dim / C::BK);
        substep(lds, 1);  // step 0, sub-step 0
        block_barrier();
        for (int kt = 0; kt + 1 < nk32; ++kt) {
            uint16_t* cur = lds + (kt & 1) * C::kStageElems;
            const uint16_t* nxt = lds + ((kt + 1) & 1) * C::kStageElems;
            const int kn = kt + 2;
#pragma unroll
            for (int i = 0; i < kMf; ++i) {
                mfma(i);
                if (i % kEvery == 0 && i / kEvery < kLoads && wave < C::kLoadWaves) {
                    if (kn < nfull) {
                        ld.issue_one(bufs, cur, kn, i / kEvery);
                    } else if constexpr (kLoop == kBufTail) {
                        if (kn < nk32)
                            ld.issue_one_tail(bufs, a_tile, g_tile, u_tile, cur, kn, i / kEvery, k_dim);
                    }
                }
                reads_after(i, nxt, 0);
                __builtin_amdgcn_sched_barrier(0);  // keep this order: MFMA, load, reads
            }
            substep(nxt, 1);  // step kt + 1, sub-step 0
            block_barrier();
        }
#pragma unroll
        for (int i = 0; i < kMf; ++i) mfma(i);  // the last step's sub-step 1
        __builtin_amdgcn_sched_barrier(0);
    } else {
        for (int64_t kt = 0; kt < nk; ++kt) {
            uint16_t* cur = lds + (kt & 1) * C::kStageElems;
            const uint16_t* nxt = lds + ((kt + 1) & 1) * C::kStageElems;
            substep(cur, 1);
            if (kt + 1 < nk) {
                block_barrier();
                if (kt + 2 < nk) ld.issue(cur, kt + 2, k_dim);
                substep(nxt, 0);
            } else {
#pragma unroll
                for (int i = 0; i < kMf; ++i) mfma(i);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
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
template <class C, Epi kEpi, bool kWriteX, int kLoop>
__global__ __launch_bounds__(C::kThreads) __attribute__((amdgpu_waves_per_eu(C::OCC))) void grouped_gemm_kernel(
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ w1, const uint16_t* __restrict__ w2,
    const int32_t* __restrict__ offs, const float* __restrict__ probs, void* __restrict__ out,
    uint16_t* __restrict__ x_out, int64_t tokens, int64_t k_dim, int64_t n_dim, int64_t experts, float L,
    int64_t n_tiles, int64_t n_blocks) {
    // One LDS object: the K-step stages (then the staging tile), followed by
    // the tile rows' probabilities. (A second __shared__ array made the
    // compiler attach alias scopes to LDS accesses, after which it no longer
    // told the main loop's fragment reads from its direct-to-LDS loads and
    // waited for every load in flight at each K step: twice the run time.)
    __shared__ __attribute__((aligned(16))) uint16_t lds[C::kLdsElems + 2 * C::BM];
    float* const ptile = reinterpret_cast<float*>(lds + C::kLdsElems);
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
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / 64);
    const int wm = wave / C::WN, wn = wave % C::WN;

    f32x4 acc_g[MI][NI], acc_u[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
            acc_g[mi][ni] = f32x4{};
            acc_u[mi][ni] = f32x4{};
        }

    // The tile rows' probabilities go straight into LDS (a direct load, one
    // dword per lane; rows past the tile repeat its last row), in flight with
    // the first K step's loads, which the main loop waits for before its first
    // barrier. The epilogue then reads them from LDS.
    if (wave < C::BM / 64) {
        const int r = wave * 64 + lane;
        __builtin_amdgcn_global_load_lds(probs + tr.row0 + (r < tr.rows ? r : tr.rows - 1),
                                         (__attribute__((address_space(3))) void*)(ptile + wave * 64), 4, 0, 0);
    }
    mainloop_pipe<C, kLoop>(lds, a_tile, g_tile, u_tile, tr.rows, ncols1, ncols2 > 0 ? ncols2 : 1, k_dim, acc_g, acc_u);
    lds_barrier();  // all fragment reads done before the buffers become the staging tile

    // Each staged output tile is written to LDS in 16-byte row chunks (eight
    // bf16 columns or four fp32 columns per lane and write, see row_chunk) and
    // read back as 16-byte row-contiguous chunks for the global stores.
    uint16_t* stage = lds;
    if constexpr (kEpi == Epi::kSwiglu) {
        uint16_t* y = static_cast<uint16_t*>(out);
        // stage one bf16 tile: pair(mi, ni, j, p) gives the outputs of registers
        // j and j + 1 of tile (mi, ni), p the probability of its row; column
        // tiles ni and ni + 1 are exchanged together (row_chunk)
        auto stage_bf16 = [&](auto&& pair) {
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const int r = acc_row<C>(wm, mi, lane);
                const float p = ptile[r];
#pragma unroll
                for (int ni = 0; ni < NI; ni += 2) {
                    const u32x4 v = row_chunk([&](int t, int j) { return pair(mi, ni + t, j, p); });
                    *reinterpret_cast<u32x4*>(stage + r * C::kLdo + acc_col<C>(wn, ni + chunk_tile(lane), 0) +
                                              chunk_col(lane)) = v;
                }
            }
        };
        stage_bf16([&](int mi, int ni, int j, float p) {
            const f32x2 g = round2_bf16(acc_g[mi][ni][j], acc_g[mi][ni][j + 1]);
            const f32x2 u = round2_bf16(acc_u[mi][ni][j], acc_u[mi][ni][j + 1]);
            return f32x2{fwd_elem(g[0], u[0], p, L), fwd_elem(g[1], u[1], p, L)};
        });
        lds_barrier();
        store_tile<C>(stage, y, n_dim, tr.row0, tr.rows, col1, n_dim);
        if constexpr (kWriteX) {
            lds_barrier();
            stage_bf16([&](int mi, int ni, int j, float) { return f32x2{acc_g[mi][ni][j], acc_g[mi][ni][j + 1]}; });
            lds_barrier();
            store_tile<C>(stage, x_out, 2 * n_dim, tr.row0, tr.rows, col1, n_dim);
            lds_barrier();
            stage_bf16([&](int mi, int ni, int j, float) { return f32x2{acc_u[mi][ni][j], acc_u[mi][ni][j + 1]}; });
            lds_barrier();
            store_tile<C>(stage, x_out + n_dim, 2 * n_dim, tr.row0, tr.rows, col1, n_dim);
        }
    } else if constexpr (kEpi == Epi::kRouterF32) {
        // fp32 staged through LDS, one weight tile (BM x BN floats, all of the
        // LDS) at a time, then stored as 16-byte row-contiguous chunks. Each
        // row's 16-byte chunks are XOR-swizzled by the row's low four bits, so
        // a wavefront's write (32 rows, one chunk each) spreads over the banks.
        // Stores straight from the accumulators ran slower: 13% with 4 bytes per
        // lane, 9% with 16 (a lane's four consecutive columns, 32 bytes of a row
        // per wavefront half and store).
        static_assert(C::BM * C::BN * 4 <= C::kLdsElems * 2, "an fp32 tile fits the LDS");
        static_assert(C::BN % 64 == 0, "the swizzle permutes chunks within 64-column groups");
        float* o = static_cast<float*>(out);
        float* stf = reinterpret_cast<float*>(lds);
        auto sw = [](int r, int c) { return c ^ ((r & 15) << 2); };
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int ncols = half == 0 ? ncols1 : ncols2;
            const int64_t colb = half == 0 ? col1 : col2;
            if (ncols == 0) break;
            if (half == 1) lds_barrier();  // the first half's stores have read the staging tile
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const int r = acc_row<C>(wm, mi, lane);
                const float p = ptile[r];
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) {
                    const f32x4& v = half == 0 ? acc_g[mi][ni] : acc_u[mi][ni];
                    const f32x2 lo = round2_bf16(v[0], v[1]), hi = round2_bf16(v[2], v[3]);
                    const f32x4 w{lo[0] * p, lo[1] * p, hi[0] * p, hi[1] * p};
                    *reinterpret_cast<f32x4*>(stf + r * C::BN + sw(r, acc_col<C>(wn, ni, lane))) = w;
                }
            }
            lds_barrier();
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
            if (half == 1) lds_barrier();  // the first half's stores have read the staging tile
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const int r = acc_row<C>(wm, mi, lane);
                const float p = ptile[r];
#pragma unroll
                for (int ni = 0; ni < NI; ni += 2) {
                    const u32x4 c = row_chunk([&](int t, int j) {
                        const f32x4& v = half == 0 ? acc_g[mi][ni + t] : acc_u[mi][ni + t];
                        const f32x2 r2 = round2_bf16(v[j], v[j + 1]);
                        return f32x2{r2[0] * p, r2[1] * p};
                    });
                    *reinterpret_cast<u32x4*>(stage + r * C::kLdo + acc_col<C>(wn, ni + chunk_tile(lane), 0) +
                                              chunk_col(lane)) = c;
                }
            }
            lds_barrier();
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
void launch_kernel(int loop, int64_t grid, hipStream_t st, const uint16_t* a, const uint16_t* w1, const uint16_t* w2,
                   const int32_t* offs, const float* probs, void* out, uint16_t* x_out, int64_t tokens, int64_t k_dim,
                   int64_t n_dim, int64_t experts, float limit, int64_t n_tiles, int64_t n_blocks) {
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(grid)), dim3(C::kThreads), 0, st, a, w1, w2, offs, probs,
                           out, x_out, tokens, k_dim, n_dim, experts, limit, n_tiles, n_blocks);
    };
    if (loop == kBufLoop)
        go(grouped_gemm_kernel<C, kEpi, kWriteX, kBufLoop>);
    else if (loop == kBufTail)
        go(grouped_gemm_kernel<C, kEpi, kWriteX, kBufTail>);
    else
        go(grouped_gemm_kernel<C, kEpi, kWriteX, kPtrLoop>);
}

template <class C, Epi kEpi>
int launch_grouped(const uint16_t* a, const uint16_t* w1, const uint16_t* w2, const int32_t* offs,
                   const float* probs, void* out, uint16_t* x_out, int64_t tokens, int64_t k_dim, int64_t n_dim,
                   int64_t experts, float limit, hipStream_t st) {
    int64_t n_tiles, n_blocks;
    const int64_t grid = grouped_grid(tokens, n_dim, kEpi == Epi::kSwiglu ? C::BN : 2 * C::BN, experts, C::BM, &n_tiles,
                                         &n_blocks);
    if (grid == 0) return MOE_EPI_ERR_BAD_SHAPE;
    const int loop = k_dim > kBufMaxK<C> ? kPtrLoop : k_dim % C::BK == 0 ? kBufLoop : kBufTail;
    (void)hipGetLastError();
    if (kEpi == Epi::kSwiglu && x_out)
        launch_kernel<C, kEpi, true>(loop, grid, st, a, w1, w2, offs, probs, out, x_out, tokens, k_dim, n_dim, experts,
                                     limit, n_tiles, n_blocks);
    else
        launch_kernel<C, kEpi, false>(loop, grid, st, a, w1, w2, offs, probs, out, x_out, tokens, k_dim, n_dim, experts,
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
