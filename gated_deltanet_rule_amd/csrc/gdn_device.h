// gdn_device.h -- device-side helpers shared by the libgdn kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Storage tag for bfloat16 tensors (raw 16-bit patterns in memory).
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t bf16_bits_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

template <typename E> __device__ __forceinline__ E from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
    bf16_t r;
    r.bits = bf16_bits_rne(x);
    return r;
}

// Wave-wide (64 lanes) sum.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

}  // namespace gdn
