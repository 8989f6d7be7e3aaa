// Shared device helpers and host-side argument checks for libmoe_epi (gfx950).
//
// Data movement: a lane moves a "vector" of 8 elements at a time (16 bytes of
// bfloat16 / float16, 32 bytes of float32) and the kernels keep several
// vectors per lane in flight. Every streamed tensor is read once and written
// once, so all vector accesses carry the nontemporal hint (the `nt`
// cache-policy bit): on MI355X this raised sustained bandwidth of these
// kernels by 10-15% over default-policy accesses (measured: SwiGLU forward
// 290 -> 249 us, backward 493 -> 446 us at 131072 x 2048 bfloat16). Vectors
// stay packed in registers until the math needs them. Which 8 elements a lane
// takes is set by the vector map (quads_of below). The per-element path
// (scalar kernels) exists for row widths that are not a multiple of 8 or
// pointers that are not 16-byte aligned.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "moe_epi.h"

namespace moe_epi {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // 8 packed 16-bit values

// ---- bfloat16 <-> float32 in registers ------------------------------------

// Widening is exact: a bfloat16 is the upper half of a float32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_at(const uint16_t* p) { return __uint_as_float(static_cast<uint32_t>(*p) << 16); }

// Two float32 -> packed bfloat16 pair with one v_cvt_pk_bf16_f32 (round to
// nearest even under the default rounding mode).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ uint16_t to_bf16(float v) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

// ---- streaming accesses -------------------------------------------------------

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));  // 4 packed 16-bit values

__device__ __forceinline__ u32x4 load_nt16(const void* p) {
    return __builtin_nontemporal_load(static_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store_nt16(void* p, u32x4 v) { __builtin_nontemporal_store(v, static_cast<u32x4*>(p)); }
__device__ __forceinline__ u32x2 load_nt8(const void* p) {
    return __builtin_nontemporal_load(static_cast<const u32x2*>(p));
}
__device__ __forceinline__ void store_nt8(void* p, u32x2 v) { __builtin_nontemporal_store(v, static_cast<u32x2*>(p)); }

// ---- the vector map ---------------------------------------------------------------
//
// A lane's vector is two quads of 4 elements, at element offsets a and b of
// the row. The G lanes of a row group walk the row in chunks of n consecutive
// vectors (n = G, fewer in the row's last chunk); vector c belongs to lane
// c % G of the chunk that starts at vector c - lane.
//  - contiguous map: vector c is elements [8c, 8c + 8) (b = a + 4); a 16-bit
//    vector is one 16-byte access, and a wavefront's access covers 1 KiB;
//  - split map: lane l's quads are elements 4l and 4n + 4l of the chunk, so
//    every wavefront-wide quad access covers one contiguous run (1 KiB of
//    float32, 512 bytes of 16-bit values). Kernels that stream a float32
//    tensor use it: under the contiguous map a float32 vector's two 16-byte
//    halves sit 32 bytes apart across the lanes of each instruction, and
//    such half-filled accesses ran at 62-70% of the bandwidth of the same
//    kernel on 16-bit data (43% with float32 stores fed by bfloat16 loads).
// Both maps cover a chunk's 8n elements exactly once.
struct Quads {
    uint32_t a, b;  // element offsets within the row
};

template <int G, bool kSplit>
__host__ __device__ __forceinline__ Quads quads_of(uint32_t c, uint32_t lane, uint32_t nvec) {
    if constexpr (kSplit) {
        const uint32_t base = c - lane;  // first vector of this chunk
        const uint32_t n = nvec - base < static_cast<uint32_t>(G) ? nvec - base : static_cast<uint32_t>(G);
        const uint32_t a = 8 * base + 4 * lane;
        return {a, a + 4 * n};
    } else {
        return {8 * c, 8 * c + 4};
    }
}

// ---- addressing -------------------------------------------------------------------
//
// Vector kernels address a row as (row base pointer, 32-bit byte offset): the
// host sends rows of 2 GiB and more to the per-element kernels, so in-row
// offsets fit in 32 bits. With a wave-uniform row (below) the base stays in
// scalar registers and each access is one global load/store with a scalar
// base and a 32-bit per-lane offset, which keeps the 64-bit address
// arithmetic, and the registers it takes, out of the vector ALU.

template <int kBytes>
__device__ __forceinline__ const void* at(const void* row, uint32_t i) {
    return static_cast<const char*>(row) + i * static_cast<uint32_t>(kBytes);
}
template <int kBytes>
__device__ __forceinline__ void* at(void* row, uint32_t i) {
    return static_cast<char*>(row) + i * static_cast<uint32_t>(kBytes);
}

// Index, within the block, of the lane group (row) the calling lane belongs
// to. With G >= 64 each wavefront lies inside one group, so the index is
// wave-uniform; readfirstlane tells the compiler so, and the row's index,
// probability and base addresses then live in scalar registers.
template <int G>
__device__ __forceinline__ int group_in_block() {
    static_assert(G < 64 || G % 64 == 0, "groups of 64 lanes or more are whole wavefronts");
    const int g = static_cast<int>(threadIdx.x) / G;
    if constexpr (G >= 64)
        return __builtin_amdgcn_readfirstlane(g);
    else
        return g;
}

// ---- aligned row loads ---------------------------------------------------------
//
// A barrier of the whole block before its wavefronts issue their row loads, so
// that the block's requests (its rows are contiguous in memory) reach the
// memory system together rather than spread over the time its wavefronts
// took to start. Every wavefront of the block must call it the same number of
// times, rows past the end included. Measured on MI355X with the caches
// flushed before every launch: the clamped SwiGLU forward at 131072 x 2048
// bf16 went from 80.8-81.0% to 85.1-85.5% of HBM peak with three 192-lane
// rows per block, the backward from 78.6% to 82.8-83.1%; a wait for the
// row's probability before the loads did the same. Blocks of 256-lane rows
// gained nothing from it.
__device__ __forceinline__ void align_block_loads() { __syncthreads(); }

// ---- occupancy ------------------------------------------------------------------
//
// Waves per SIMD that let two blocks of B threads share a CU: a block's waves
// are spread over the CU's 4 SIMDs, so each SIMD needs room for
// ceil(B / 256) waves per block. Given to amdgpu_waves_per_eu, this caps the
// kernel's registers (at 8 waves, 64 VGPRs) instead of leaving the occupancy
// to how the compiler happens to schedule the math: the router backward at
// 448 lanes per row dropped from 79.7% to 75.2% of HBM bandwidth when its
// VGPRs went from 54 to 66 and a CU held one 896-thread block instead of two.
constexpr int waves_for_two_blocks(int B) {
    const int w = 2 * ((B + 255) / 256);
    return w > 8 ? 8 : w;
}

// ---- element types: 8 elements per vector ------------------------------------
//
// Elem<T> moves a vector of storage type T (load / store at row offset `row`,
// quads q), widens it to float32 (unpack: quad a gives f[0..3], quad b
// f[4..7]) and rounds float32 back to T (pack: round to nearest even; float32
// is stored as is). load1 / store1 are the per-element forms.

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// 16-bit storage: Raw holds quad a in words 0-1 and quad b in words 2-3.
struct Bits16 {
    using Raw = u32x4;
    static constexpr int kBytes = 2;
    template <bool kSplit>
    __device__ __forceinline__ static Raw load(const void* row, Quads q) {
        if constexpr (kSplit) {
            const u32x2 a = load_nt8(at<2>(row, q.a)), b = load_nt8(at<2>(row, q.b));
            return Raw{a[0], a[1], b[0], b[1]};
        } else {
            return load_nt16(at<2>(row, q.a));
        }
    }
    template <bool kSplit>
    __device__ __forceinline__ static void store(void* row, Quads q, Raw v) {
        if constexpr (kSplit) {
            store_nt8(at<2>(row, q.a), u32x2{v[0], v[1]});
            store_nt8(at<2>(row, q.b), u32x2{v[2], v[3]});
        } else {
            store_nt16(at<2>(row, q.a), v);
        }
    }
};

template <int T> struct Elem;

template <> struct Elem<MOE_EPI_BF16> : Bits16 {
    __device__ __forceinline__ static void unpack(Raw r, float (&f)[8]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f[2 * k] = bf16_lo(r[k]);
            f[2 * k + 1] = bf16_hi(r[k]);
        }
    }
    __device__ __forceinline__ static Raw pack(const float (&f)[8]) {
        Raw r;
#pragma unroll
        for (int k = 0; k < 4; ++k) r[k] = pack_bf16x2(f[2 * k], f[2 * k + 1]);
        return r;
    }
    __device__ __forceinline__ static float load1(const void* p, int64_t i) {
        return bf16_at(static_cast<const uint16_t*>(p) + i);
    }
    __device__ __forceinline__ static void store1(void* p, int64_t i, float v) {
        static_cast<uint16_t*>(p)[i] = to_bf16(v);
    }
};

template <> struct Elem<MOE_EPI_F16> : Bits16 {
    // Each 32-bit word is taken out of the vector as a scalar first: bit-casting
    // a vector element straight to a two-lane half vector was compiled by this
    // hipcc as if every element were element 0 (seen in the gfx950 ISA).
    __device__ __forceinline__ static void unpack(Raw r, float (&f)[8]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t w = r[k];
            f[2 * k] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xFFFFu)));
            f[2 * k + 1] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
        }
    }
    __device__ __forceinline__ static Raw pack(const float (&f)[8]) {
        Raw r;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const f32x2_t w = {f[2 * k], f[2 * k + 1]};
            r[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(w, f16x2_t));
        }
        return r;
    }
    __device__ __forceinline__ static float load1(const void* p, int64_t i) {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<const uint16_t*>(p)[i]));
    }
    // The empty asm pins v as a finished binary32 value. Without it this hipcc
    // folds a product feeding the cast into one mixed-precision fma with a +0
    // addend and a half result: that rounds the exact product once (not the
    // binary32 product, then to half) and turns a -0 product into +0.
    __device__ __forceinline__ static void store1(void* p, int64_t i, float v) {
        asm volatile("" : "+v"(v));
        static_cast<uint16_t*>(p)[i] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
    }
};

// float32 storage: each quad is one 16-byte access under either map.
template <> struct Elem<MOE_EPI_F32> {
    struct Raw {
        u32x4 a, b;
    };
    static constexpr int kBytes = 4;
    template <bool kSplit>
    __device__ __forceinline__ static Raw load(const void* row, Quads q) {
        return Raw{load_nt16(at<4>(row, q.a)), load_nt16(at<4>(row, q.b))};
    }
    template <bool kSplit>
    __device__ __forceinline__ static void store(void* row, Quads q, Raw v) {
        store_nt16(at<4>(row, q.a), v.a);
        store_nt16(at<4>(row, q.b), v.b);
    }
    __device__ __forceinline__ static void unpack(Raw r, float (&f)[8]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f[k] = __uint_as_float(r.a[k]);
            f[4 + k] = __uint_as_float(r.b[k]);
        }
    }
    __device__ __forceinline__ static Raw pack(const float (&f)[8]) {
        Raw r;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            r.a[k] = __float_as_uint(f[k]);
            r.b[k] = __float_as_uint(f[4 + k]);
        }
        return r;
    }
    __device__ __forceinline__ static float load1(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
    __device__ __forceinline__ static void store1(void* p, int64_t i, float v) { static_cast<float*>(p)[i] = v; }
};

// Base pointer of the row that starts at element offset i of a tensor of T.
template <int T>
__device__ __forceinline__ const void* row_at(const void* p, int64_t i) {
    return static_cast<const char*>(p) + i * Elem<T>::kBytes;
}
template <int T>
__device__ __forceinline__ void* row_at(void* p, int64_t i) {
    return static_cast<char*>(p) + i * Elem<T>::kBytes;
}

inline int elem_bytes(int dtype) { return dtype == MOE_EPI_F32 ? 4 : 2; }
inline bool dtype_ok(int dtype) { return dtype == MOE_EPI_BF16 || dtype == MOE_EPI_F16 || dtype == MOE_EPI_F32; }

// Sum over the G lanes of an aligned lane group (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, G);
    return v;
}

// Sum of v over the G lanes of each row group of a block. G <= 64: the lanes of
// one wavefront (shuffles only). G > 64 (a multiple of 64): each wavefront's
// shuffle sum goes to LDS (`part`, one slot per wavefront of the block) and
// the row's partial sums are added in a fixed order, so the result does not
// depend on timing. With G > 64 every thread of the block must make the call
// (it holds two barriers).
template <int G>
__device__ __forceinline__ float row_sum(float v, float* part) {
    if constexpr (G <= 64) {
        return group_sum<G>(v);
    } else {
        v = group_sum<64>(v);
        if ((threadIdx.x & 63) == 0) part[threadIdx.x / 64] = v;
        __syncthreads();
        const int first = (threadIdx.x / G) * (G / 64);
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < G / 64; ++q) s += part[first + q];
        __syncthreads();
        return s;
    }
}

// ---- launch shapes ------------------------------------------------------------

// A launch shape: G lanes own one row (G <= 64 within a wavefront, or 64*W
// for W wavefronts per row), each lane handles V 16-byte vectors per pass over
// the row (the kernels loop over passes, so any V covers any row), and blocks
// have B threads (B / G rows per block).
// Lanes per row for rows narrower than a wavefront.
inline int small_group(int64_t nvec) { return nvec > 16 ? 32 : (nvec > 8 ? 16 : 8); }

// Grid size for a row loop: one lane group per row, capped (a grid must stay
// below 2^32 work-items) so that larger inputs are covered by the row loop.
constexpr int64_t kMaxBlocks = 1 << 20;

inline unsigned grid_for_rows(int64_t rows, int rows_per_block) {
    int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
    if (blocks > kMaxBlocks) blocks = kMaxBlocks;
    if (blocks < 1) blocks = 1;
    return static_cast<unsigned>(blocks);
}

// ---- host-side checks -------------------------------------------------------

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

inline Range range_of(const void* p, int64_t bytes) {
    uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + static_cast<uintptr_t>(bytes)};
}

inline bool overlaps(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

// rows * cols * elem_bytes must fit in int64 (and in the address space).
inline bool bytes_ok(int64_t rows, int64_t cols, int64_t elem_bytes, int64_t* out) {
    if (rows < 0 || cols <= 0) return false;
    const int64_t lim = INT64_MAX / 4;
    if (rows != 0 && cols > lim / elem_bytes / rows) return false;
    *out = rows * cols * elem_bytes;
    return true;
}

// The vector kernels take in-row byte offsets in 32 bits.
inline bool row_fits_u32_offsets(int64_t cols, int elem_bytes) {
    return cols <= (static_cast<int64_t>(1) << 31) / elem_bytes - 1;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int launch_status() {
    return hipGetLastError() == hipSuccess ? MOE_EPI_SUCCESS : MOE_EPI_ERR_LAUNCH;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace moe_epi
