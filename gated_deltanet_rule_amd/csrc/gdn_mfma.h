// gdn_mfma.h -- 16x16 matrix-core tiles for gfx950 (CDNA4), wave64.
//
// Every product here is built from one instruction family per element type:
//   bf16: v_mfma_f32_16x16x32_bf16  (8 bf16 per lane for A and B, K = 32)
//   fp32: v_mfma_f32_16x16x4_f32    (1 fp32 per lane, K = 4; issued 4 times
//                                    to cover a 16-deep K block)
// Accumulator layout (both): lane l holds column n = l % 16 and rows
// 4*(l/16) + j, j = 0..3, of the 16x16 tile.
//
// K-block convention.  Within a K block of KB rows (32 for bf16, 16 for
// fp32), lane l = 16*qd + m supplies the k-offsets
//     bf16: 4*qd + j and 16 + 4*qd + j   (j = 0..3; 8 values)
//     fp32: 4*qd + j                     (j = 0..3; one per instruction)
// for both operands.  A dot product does not care which k goes to which
// hardware slot as long as A and B agree, and with this choice the B operand
// of a K block is exactly what a lane already holds in the accumulator
// tiles covering those KB rows (two tiles for bf16, one for fp32).  A state
// or value matrix produced by one product can therefore feed the next
// product straight from registers, with no LDS round trip.
#pragma once

#include "gdn_device.h"

namespace gdn {

template <typename E> struct Mfma;

template <> struct Mfma<bf16_t> {
    static constexpr int KB = 32;
    using Frag = bf16x8;

    __device__ static __forceinline__ void mma(floatx4 &c, const Frag &a, const Frag &b) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // operand from a row-major bf16 matrix: `row` points at the lane's row
    __device__ static __forceinline__ Frag load_rm(const bf16_t *row, int k0, int qd) {
        const uint2 lo = *reinterpret_cast<const uint2 *>(row + k0 + 4 * qd);
        const uint2 hi = *reinterpret_cast<const uint2 *>(row + k0 + 16 + 4 * qd);
        const uint4 u = make_uint4(lo.x, lo.y, hi.x, hi.y);
        return __builtin_bit_cast(Frag, u);
    }
    // operand from a row-major fp32 matrix, each k scaled by ks[k] (LDS)
    __device__ static __forceinline__ Frag load_rm_f32(const float *row, int k0, int qd,
                                                        const float *ks) {
        const float4 lo = *reinterpret_cast<const float4 *>(row + k0 + 4 * qd);
        const float4 hi = *reinterpret_cast<const float4 *>(row + k0 + 16 + 4 * qd);
        const float4 sl = *reinterpret_cast<const float4 *>(ks + k0 + 4 * qd);
        const float4 sh = *reinterpret_cast<const float4 *>(ks + k0 + 16 + 4 * qd);
        Frag f;
        f[0] = (__bf16)(lo.x * sl.x); f[1] = (__bf16)(lo.y * sl.y);
        f[2] = (__bf16)(lo.z * sl.z); f[3] = (__bf16)(lo.w * sl.w);
        f[4] = (__bf16)(hi.x * sh.x); f[5] = (__bf16)(hi.y * sh.y);
        f[6] = (__bf16)(hi.z * sh.z); f[7] = (__bf16)(hi.w * sh.w);
        return f;
    }
    // B operand of K block kb from accumulator tiles t[2kb], t[2kb+1], times s
    __device__ static __forceinline__ Frag from_acc(const floatx4 *t, int kb, float s) {
        const floatx4 lo = t[2 * kb], hi = t[2 * kb + 1];
        Frag f;
        f[0] = (__bf16)(lo[0] * s); f[1] = (__bf16)(lo[1] * s);
        f[2] = (__bf16)(lo[2] * s); f[3] = (__bf16)(lo[3] * s);
        f[4] = (__bf16)(hi[0] * s); f[5] = (__bf16)(hi[1] * s);
        f[6] = (__bf16)(hi[2] * s); f[7] = (__bf16)(hi[3] * s);
        return f;
    }
    // number of 16-row accumulator tiles per K block
    static constexpr int TPB = 2;
};

template <> struct Mfma<float> {
    static constexpr int KB = 16;
    using Frag = floatx4;

    __device__ static __forceinline__ void mma(floatx4 &c, const Frag &a, const Frag &b) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    }
    __device__ static __forceinline__ Frag load_rm(const float *row, int k0, int qd) {
        const float4 v = *reinterpret_cast<const float4 *>(row + k0 + 4 * qd);
        Frag f = {v.x, v.y, v.z, v.w};
        return f;
    }
    __device__ static __forceinline__ Frag load_rm_f32(const float *row, int k0, int qd,
                                                        const float *ks) {
        const float4 v = *reinterpret_cast<const float4 *>(row + k0 + 4 * qd);
        const float4 s = *reinterpret_cast<const float4 *>(ks + k0 + 4 * qd);
        Frag f = {v.x * s.x, v.y * s.y, v.z * s.z, v.w * s.w};
        return f;
    }
    __device__ static __forceinline__ Frag from_acc(const floatx4 *t, int kb, float s) {
        const floatx4 v = t[kb];
        Frag f = {v[0] * s, v[1] * s, v[2] * s, v[3] * s};
        return f;
    }
    static constexpr int TPB = 1;
};

// Two-term operands.  A bf16 operand carries 8 significant bits; the WY
// factors, the masked attention, the state and the chunk deltas are fp32
// quantities, so each is passed to the matrix cores as hi + lo with
// hi = bf16(x), lo = bf16(x - hi) (about 16 significant bits together), and
// a product X*Y becomes X_hi*Y + X_lo*Y (or three terms when both sides are
// split).  Inputs q, k, v are exact in bf16 and never need a second term.
// With fp32 operands there is nothing to split (SPLIT == 1).
template <typename E> struct Split;
template <> struct Split<bf16_t> {
    static constexpr int N = 2;
    using Frag = bf16x8;
    __device__ static __forceinline__ void acc(const floatx4 *t, int kb, float s, Frag &hi, Frag &lo) {
        const floatx4 a = t[2 * kb], b = t[2 * kb + 1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float x = a[j] * s, y = b[j] * s;
            const __bf16 xh = (__bf16)x, yh = (__bf16)y;
            hi[j] = xh;
            hi[4 + j] = yh;
            lo[j] = (__bf16)(x - (float)xh);
            lo[4 + j] = (__bf16)(y - (float)yh);
        }
    }
    __device__ static __forceinline__ void rm_f32(const float *row, int k0, int qd, const float *ks,
                                                  Frag &hi, Frag &lo) {
        const float4 l = *reinterpret_cast<const float4 *>(row + k0 + 4 * qd);
        const float4 h = *reinterpret_cast<const float4 *>(row + k0 + 16 + 4 * qd);
        const float4 sl = *reinterpret_cast<const float4 *>(ks + k0 + 4 * qd);
        const float4 sh = *reinterpret_cast<const float4 *>(ks + k0 + 16 + 4 * qd);
        const float v[8] = {l.x * sl.x, l.y * sl.y, l.z * sl.z, l.w * sl.w,
                            h.x * sh.x, h.y * sh.y, h.z * sh.z, h.w * sh.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const __bf16 b = (__bf16)v[j];
            hi[j] = b;
            lo[j] = (__bf16)(v[j] - (float)b);
        }
    }
};
template <> struct Split<float> {
    static constexpr int N = 1;
    using Frag = floatx4;
    __device__ static __forceinline__ void acc(const floatx4 *t, int kb, float s, Frag &hi, Frag &lo) {
        hi = Mfma<float>::from_acc(t, kb, s);
        lo = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    __device__ static __forceinline__ void rm_f32(const float *row, int k0, int qd, const float *ks,
                                                  Frag &hi, Frag &lo) {
        hi = Mfma<float>::load_rm_f32(row, k0, qd, ks);
        lo = floatx4{0.f, 0.f, 0.f, 0.f};
    }
};

// Fragments live in memory as 64 lanes x 16 bytes (1 KiB), lane-major, so a
// wave moves one with a single fully coalesced 16-byte access per lane.
template <typename E>
__device__ __forceinline__ typename Mfma<E>::Frag load_frag(const void *base, int f, int lane) {
    const uint4 u = *(reinterpret_cast<const uint4 *>(base) + (size_t)f * 64 + lane);
    return __builtin_bit_cast(typename Mfma<E>::Frag, u);
}
template <typename E>
__device__ __forceinline__ void store_frag(void *base, int f, int lane, const typename Mfma<E>::Frag &v) {
    *(reinterpret_cast<uint4 *>(base) + (size_t)f * 64 + lane) = __builtin_bit_cast(uint4, v);
}

// fp32 16x16x16 product step on fp32 operands (used by the triangular
// inverse in both element types): c += A(16x16 at a_row, k0..k0+15) * B where
// the B operand is given per lane as 4 fp32 values for k = 4*qd + j.
__device__ __forceinline__ void mma_f32_k16(floatx4 &c, const floatx4 &a, const floatx4 &b) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
}

}  // namespace gdn
