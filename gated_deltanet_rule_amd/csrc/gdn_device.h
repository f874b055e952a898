// gdn_device.h -- device-side helpers shared by the libgdn kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // raw 16-byte word
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

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
    r.bits = __builtin_bit_cast(uint16_t, (__bf16)x);   // v_cvt_pk_bf16_f32: round to nearest even
    return r;
}

// Raw buffer resource over `bytes` bytes at `base`: stores at offsets past
// the end are dropped by the hardware range check, which lets a partial tile
// be written without a branch per row (a branch around a store leaves the
// compiler unable to count it, and the next wait for a load then waits for
// the store too).  0x00020000 is the gfx9 dword-3 value of a raw 32-bit
// buffer.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void buffer_store(float v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}
__device__ __forceinline__ void buffer_store(bf16_t v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b16(v.bits, r, off, 0, 0);
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// waits for every outstanding global load and store of the wave, which would
// serialise a prefetch issued before the barrier with the barrier itself.
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The layer's gate activations, raw projections -> operator inputs:
// beta = sigmoid(b) and g = softplus(a + bias) * rate, with softplus(x) =
// log(1 + e^x) evaluated as max(x, 0) + log1p(e^-|x|) so that nothing
// overflows.  `raw` selects them; otherwise a and b pass through unchanged.
struct Gates {
    const float *rate;     // [H_v] decay rate (<= 0)
    const float *bias;     // [H_v] gate bias
    int raw;
};
__device__ __forceinline__ float gate_g(float a, float bias, float rate) {
    const float x = a + bias;
    return (fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)))) * rate;
}
__device__ __forceinline__ float gate_beta(float b) { return 1.f / (1.f + expf(-b)); }

// silu(x) = x * sigmoid(x) = x / (1 + e^-x) (e^-x overflowing to inf gives -0).
__device__ __forceinline__ float silu(float x) { return x / (1.f + expf(-x)); }

// Wave-wide (64 lanes) sum.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

}  // namespace gdn
