// bf16_split.h -- bf16 operand splits for fp32 values that enter bf16
// MFMAs: x = hi + lo (two terms, ~2^-17 relative) or hi + mid + lo (three
// terms, ~2^-26), and the k-block operand built from an accumulator pair.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Splits work on pairs: one packed conversion gives both bf16 (round to
// nearest even), and their float values are a shift and a mask of it.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}
__device__ __forceinline__ float pk_first(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float pk_second(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// (a, b) = hi + lo: hi = bf16(x), lo = bf16(x - hi), as packed pairs
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = pk_bf16(a, b);
    lo = pk_bf16(a - pk_first(hi), b - pk_second(hi));
}

// hi = bf16(x), lo = bf16(x - hi)
__device__ __forceinline__ void split4(const f32x4 &x, bf16x4 &hi, bf16x4 &lo) {
    uint32_t h0, l0, h1, l1;
    split2(x[0], x[1], h0, l0);
    split2(x[2], x[3], h1, l1);
    hi = __builtin_bit_cast(bf16x4, (u32x2{h0, h1}));
    lo = __builtin_bit_cast(bf16x4, (u32x2{l0, l1}));
}

// three-term split: x = hi + mid + lo to ~2^-26 relative
__device__ __forceinline__ void split3(const f32x4 &x, bf16x4 &hi, bf16x4 &mid, bf16x4 &lo) {
    uint32_t h[2], m[2], o[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        h[j] = pk_bf16(x[2 * j], x[2 * j + 1]);
        const float r0 = x[2 * j] - pk_first(h[j]), r1 = x[2 * j + 1] - pk_second(h[j]);
        split2(r0, r1, m[j], o[j]);
    }
    hi = __builtin_bit_cast(bf16x4, (u32x2{h[0], h[1]}));
    mid = __builtin_bit_cast(bf16x4, (u32x2{m[0], m[1]}));
    lo = __builtin_bit_cast(bf16x4, (u32x2{o[0], o[1]}));
}

// k-block operand from an accumulator pair (rows 32j+4g+e, 32j+16+4g+e)
__device__ __forceinline__ void pair_operand(const f32x4 &t0, const f32x4 &t1, bf16x8 &hi, bf16x8 &lo) {
    bf16x4 h0, l0, h1, l1;
    split4(t0, h0, l0);
    split4(t1, h1, l1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        hi[i] = h0[i];
        hi[4 + i] = h1[i];
        lo[i] = l0[i];
        lo[4 + i] = l1[i];
    }
}


}  // namespace
}  // namespace hla
