// Device helpers shared by the libmilo kernels (gfx950 / CDNA4 only).
//
// MFMA operand layouts used throughout (wave64):
//   v_mfma_f32_32x32x16_bf16: lane l supplies A[m = l%32][k = 8*(l/32) + e] and
//     B[k = 8*(l/32) + e][n = l%32] for e = 0..7; it receives
//     C[m = 8*(i/4) + 4*(l/32) + i%4][n = l%32] in accumulator i = 0..15.
//   v_mfma_f32_16x16x32_bf16: lane l supplies A[m = l%16][k = 8*(l/16) + e] and
//     B[k = 8*(l/16) + e][n = l%16]; it receives C[m = 4*(l/16) + i][n = l%16],
//     i = 0..3.
// Because a contraction only needs A and B to agree on which k each slot
// holds, kernels freely permute k inside a step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace milo {

constexpr int kD = 128;  // head_dim supported by every kernel

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (NaN stays NaN): one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two values in one conversion: low half = a, high half = b.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_bits(float a, float b) {
    typedef float f2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
    const f2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2_t));
}

// Exact split of an fp32 value into three bf16 terms: f = hi + mid + lo for
// every normal f whose terms stay normal (8 + 8 + 8 significant bits).
__device__ __forceinline__ void split3_bf16(float f, uint16_t &hi, uint16_t &mid, uint16_t &lo) {
    hi = f32_to_bf16_bits(f);
    float r1 = f - bf16_bits_to_f32(hi);
    mid = f32_to_bf16_bits(r1);
    float r2 = r1 - bf16_bits_to_f32(mid);
    lo = f32_to_bf16_bits(r2);
}

__device__ __forceinline__ f32x16_t mfma32x32x16(const u16x8_t &a, const u16x8_t &b,
                                                 const f32x16_t &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma16x16x32(const u16x8_t &a, const u16x8_t &b,
                                                const f32x4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// LDS transpose read of 16-bit data (ds_read_b64_tr_b16, gfx950).  Within each
// group of 16 lanes, lane j receives element j % 4 of the 8-byte chunks that
// lanes 4e + j / 4 (e = 0..3) of its group address.  So if lane j of a group
// addresses row r0 + j / 4, columns 4 (j % 4) .. 4 (j % 4) + 3 of a row-major
// 16-bit matrix, lane j receives column j, rows r0 .. r0 + 3: four consecutive
// k values of one column of an MFMA operand, read from a k-major layout.
__device__ __forceinline__ u16x4_t lds_read_tr16(const void *p) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)(p));
    return __builtin_bit_cast(u16x4_t, v);
}

__device__ __forceinline__ u16x8_t cat8(const u16x4_t &a, const u16x4_t &b) {
    return u16x8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ f32x16_t zero16() {
    f32x16_t z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

__device__ __forceinline__ f32x4_t zero4() {
    f32x4_t z;
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = 0.f;
    return z;
}

// Reductions over the 32 lanes of one half of a wave64 (xor offsets < 32 never
// cross halves).
__device__ __forceinline__ float half_max(float v) {
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float half_sum(float v) {
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

}  // namespace milo
