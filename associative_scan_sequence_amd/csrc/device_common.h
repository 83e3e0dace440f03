// device_common.h -- small device helpers used by the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hla {

// Element loads that widen the input type to fp32 (bf16 -> fp32 is exact:
// the bf16 bits are the top half of the fp32 word).
template <typename T>
struct Elem;

template <>
struct Elem<float> {
    static __device__ __forceinline__ float get(const float *p, size_t i) { return p[i]; }
};

template <>
struct Elem<uint16_t> {
    static __device__ __forceinline__ float get(const uint16_t *p, size_t i) {
        return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
    }
};

// g^e for a small non-negative integer exponent; exactly 1 for e == 0 or g == 1.
__device__ __forceinline__ float gpow(float g, int e) {
    if (e == 0 || g == 1.0f) return 1.0f;
    return powf(g, static_cast<float>(e));
}

}  // namespace hla
