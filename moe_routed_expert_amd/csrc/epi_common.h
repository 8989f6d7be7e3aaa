// Shared device helpers and host-side argument checks for libmoe_epi (gfx950).
//
// Data movement: a "vector" is 8 bfloat16 values = 16 bytes, moved with one
// global_load_dwordx4 / global_store_dwordx4 per lane, so a 64-lane wavefront
// touches 1 KiB of contiguous memory per access. The per-element path
// (W = 1) exists for row widths that are not a multiple of 8 or pointers that
// are not 16-byte aligned.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "moe_epi.h"

namespace moe_epi {

constexpr int kBlock = 256;  // 4 wavefronts of 64 lanes

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// ---- bfloat16 <-> float32 in registers ------------------------------------

// Widening is exact: a bfloat16 is the upper half of a float32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two float32 -> packed bfloat16 pair with one v_cvt_pk_bf16_f32 (round to
// nearest even under the default rounding mode).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ uint16_t to_bf16(float v) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

// ---- W-wide bfloat16 loads and stores --------------------------------------

template <int W> struct Io;

template <> struct Io<8> {
    __device__ __forceinline__ static void load(const uint16_t* __restrict__ p, float (&f)[8]) {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
        f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
        f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
        f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
    }
    __device__ __forceinline__ static void store(uint16_t* __restrict__ p, const float (&f)[8]) {
        uint4 v;
        v.x = pack_bf16x2(f[0], f[1]);
        v.y = pack_bf16x2(f[2], f[3]);
        v.z = pack_bf16x2(f[4], f[5]);
        v.w = pack_bf16x2(f[6], f[7]);
        *reinterpret_cast<uint4*>(p) = v;
    }
};

template <> struct Io<1> {
    __device__ __forceinline__ static void load(const uint16_t* __restrict__ p, float (&f)[1]) {
        f[0] = __uint_as_float(static_cast<uint32_t>(*p) << 16);
    }
    __device__ __forceinline__ static void store(uint16_t* __restrict__ p, const float (&f)[1]) {
        *p = to_bf16(f[0]);
    }
};

// Sum over the G lanes of an aligned lane group (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, G);
    return v;
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

// elems * elem_bytes must fit in int64 (and in the address space).
inline bool bytes_ok(int64_t rows, int64_t cols, int64_t elem_bytes, int64_t* out) {
    if (rows < 0 || cols <= 0) return false;
    const int64_t lim = INT64_MAX / 4;
    if (rows != 0 && cols > lim / elem_bytes / rows) return false;
    *out = rows * cols * elem_bytes;
    return true;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int launch_status() {
    return hipGetLastError() == hipSuccess ? MOE_EPI_SUCCESS : MOE_EPI_ERR_LAUNCH;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Grid size for a row loop: one lane group per row, capped so that a resident
// grid strides over the remaining rows.
inline unsigned grid_for_rows(int64_t rows, int groups_per_block, int64_t max_blocks) {
    int64_t blocks = (rows + groups_per_block - 1) / groups_per_block;
    if (blocks > max_blocks) blocks = max_blocks;
    if (blocks < 1) blocks = 1;
    return static_cast<unsigned>(blocks);
}

}  // namespace moe_epi
