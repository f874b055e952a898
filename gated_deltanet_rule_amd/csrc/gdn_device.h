// gdn_device.h -- device-side helpers shared by the libgdn kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // raw 16-byte word
typedef unsigned int u32x3 __attribute__((ext_vector_type(3)));   // raw 12-byte word
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));   // raw 8-byte word
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
// A buffer offset past every range used here: a load from it reads zero and
// a store to it is dropped (a lane that must not access memory gets this
// offset instead of a branch around the access).
constexpr uint32_t kDropOffset = 0x80000000u;
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

// silu(x) = x * sigmoid(x) = x / (1 + e^-x), with the hardware's 2^x and
// reciprocal (each within about 1 ulp; e^-x overflowing to inf gives -0).  The
// IEEE expf and division cost about 25 instructions where these cost 5, and
// the prologue evaluates it for every channel of every row; its results feed
// operands of at most 16 significant bits.
__device__ __forceinline__ float silu(float x) {
    return x * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}

// x plus the x of the lane that the DPP control CTRL selects (every lane of
// the wave active and every source lane inside the wave).
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}

// x plus the x of the lane ROWS x 16 lanes away (ROWS 1 or 2), by the gfx950
// row swaps: with both operands x, the two results hold x and the partner
// rows' x in complementary rows, so their sum is the pair's sum in the same
// order on both sides.  The results pass through an empty asm: with
// identical operands the compiler otherwise takes the two results for one.
template <int ROWS>
__device__ __forceinline__ float row_swap_add(float x) {
    const unsigned a = __float_as_uint(x);
    unsigned lo, hi;
    if constexpr (ROWS == 1) {
        const auto r = __builtin_amdgcn_permlane16_swap(a, a, false, false);
        lo = r[0]; hi = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(a, a, false, false);
        lo = r[0]; hi = r[1];
    }
    asm volatile("" : "+v"(lo), "+v"(hi));
    return __uint_as_float(lo) + __uint_as_float(hi);
}

// Sum over aligned groups of N consecutive lanes (N a power of two, 2 to 64);
// every lane of a group receives the group's total, bitwise the same on each.
// Each step pairs a lane with one whose partial it does not hold yet: lane ^ 1
// and lane ^ 2 (quad permutations), lane 7 - i and 15 - i within a row (the
// half-row and row mirrors), then the row swaps.  All of it is VALU work: no
// LDS round trip per step, as a shuffle through ds_bpermute would take.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N >= 2 && N <= 64 && (N & (N - 1)) == 0, "group of 2 to 64 lanes");
    x = dpp_add<0xB1>(x);                               // quad_perm [1,0,3,2]
    if constexpr (N >= 4) x = dpp_add<0x4E>(x);         // quad_perm [2,3,0,1]
    if constexpr (N >= 8) x = dpp_add<0x141>(x);        // row_half_mirror
    if constexpr (N >= 16) x = dpp_add<0x140>(x);       // row_mirror
    if constexpr (N >= 32) x = row_swap_add<1>(x);
    if constexpr (N >= 64) x = row_swap_add<2>(x);
    return x;
}

}  // namespace gdn
