// Device-side building blocks shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

constexpr int kD = 512;           // head dimension, fixed by the op
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2 v = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16).
// Lane l supplies A row (l%16) and B column (l%16), each with the 8 reduction
// elements of group l/16; the accumulator lane l holds column l%16, rows
// 4*(l/16) .. 4*(l/16)+3.
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ bool valid_row(int r, int num_kv) {
    return (unsigned)r < (unsigned)num_kv;
}

template <typename T>
__device__ __forceinline__ T wave_xor(T v, int mask) {
    return __shfl_xor(v, mask, 64);
}

// Reductions over the four 16-lane rows (lanes l, l^16, l^32, l^48), with the
// gfx950 row swaps instead of LDS permutes: a 16-row swap of v with itself
// leaves rows (0,0,2,2) in one result and (1,1,3,3) in the other, a 32-lane
// swap the halves (lo,lo) and (hi,hi).  Every lane gets the same value; the
// sum is (v0 + v1) + (v2 + v3) or its mirror, equal bit for bit.
__device__ __forceinline__ float max_over_rows(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_rows(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float m = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}


// An MFMA accumulator or fragment lane c16 + 16g holds 8 bytes of row c16 at
// chunk g, so a store in that lane order puts four rows in every quad of
// lanes (measured on gfx950: 8 B/clk per CU, against 30 for quad-contiguous
// rows).  to_quad_rows moves the value to lane 4*c16 + g, so each quad stores
// one row's 32 contiguous bytes; the caller's store address must follow.
__device__ __forceinline__ u32x2 to_quad_rows(u32x2 v, int lane) {
    const int addr = 4 * ((lane >> 2) + 16 * (lane & 3));   // source lane c16 + 16g of lane 4*c16 + g
    return u32x2{(uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v[0]),
                 (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v[1])};
}

}  // namespace smla
