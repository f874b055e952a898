// gdn_layer.hip -- the two small passes of the layer fusion that do not live
// inside the operator's kernels (build_layer_attn_linear_core on the page
// "ik_llama.cpp src/llama-delta-net.cpp"):
//
//   conv_state_kernel: the new convolution state of each sequence, i.e. the
//     last kConv - 1 rows of (old state ++ the sequence's rows), per channel
//     (the page's new_conv_states view of the ssm_conv result).  It is its own
//     launch, after every kernel that read the old state, so that the state
//     can be updated in place: with H_v / H_k other than 1 or 2 a key head's
//     channels are read by several workgroups of the recurrent kernels, and
//     none of them could know when the others are done with the old values.
//     (The chunked prefill's scan and the recurrent kernels at ratios 1 and 2
//     replace the state themselves.)
//   gated_norm_kernel: out = o / sqrt(mean(o^2) + eps) * norm_w * silu(z)
//     over every (token, value head) row of the chunked prefill's fp32 o (its
//     scan spreads a row's columns over several workgroups; the recurrent
//     kernels apply the same step before o leaves the chip).  o is fp32 in
//     place in an fp32 output, else staged in the workspace, so the result
//     is rounded once.
//
// Both are HBM streams with no reuse: plain coalesced loads, one pass.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kH = kConv - 1;   // convolution state per channel

// One thread per (sequence, channel).  Sequence rows: cu[i]..cu[i+1] (clamped
// into [0, T]), or all T rows (single_T >= 0), or row i (cu null).
template <typename E>
__global__ __launch_bounds__(256) void conv_state_kernel(
    const E *__restrict__ x, int64_t T, int C, const float *conv_in, float *conv_out,
    int64_t slot_stride, const int32_t *__restrict__ cu, int single_T,
    const int32_t *__restrict__ slot_in, const int32_t *__restrict__ slot_out, int cblocks)
{
    const int i = blockIdx.x / cblocks;
    const int c = (blockIdx.x % cblocks) * 256 + threadIdx.x;
    if (c >= C) return;
    int64_t tb, te;
    if (single_T >= 0) {
        tb = 0;
        te = single_T;
    } else if (cu) {
        tb = min(max((int64_t)cu[i], (int64_t)0), T);
        te = min(max((int64_t)cu[i + 1], tb), T);
    } else {
        tb = i;
        te = i + 1;
    }
    const int sout = slot_out[i];
    if (sout < 0) return;
    const int sin = conv_in ? slot_in[i] : -1;
    float u[kH];
#pragma unroll
    for (int m = 0; m < kH; ++m)
        u[m] = sin >= 0 ? conv_in[(int64_t)sin * slot_stride + (int64_t)c * kH + m] : 0.f;
    const int64_t len = te - tb;
    float nu[kH];
#pragma unroll
    for (int j = 0; j < kH; ++j) {
        // element len + j of (state ++ rows)
        const int64_t e = len + j;
        nu[j] = e < kH ? u[e] : to_f32(x[(tb + e - kH) * C + c]);
    }
    float *o = conv_out + (int64_t)sout * slot_stride + (int64_t)c * kH;
#pragma unroll
    for (int j = 0; j < kH; ++j) o[j] = nu[j];
}

// DV / 4 lanes per row, four columns each; 256 / (DV / 4) rows per workgroup.
template <int DV, typename OT, typename ZT>
__global__ __launch_bounds__(256) void gated_norm_kernel(
    const float *o_in, OT *out, const ZT *__restrict__ z, const float *__restrict__ w, int64_t rows, float eps)
{
    constexpr int LPR = DV / 4;
    constexpr int RPB = 256 / LPR;
    const int lane = threadIdx.x % LPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    const bool live = row < rows;
    const int64_t r = live ? row : rows - 1;        // clamped: loads stay in range
    OT *op = out + r * DV + 4 * lane;
    const ZT *zp = z + r * DV + 4 * lane;
    const float4 ov = *reinterpret_cast<const float4 *>(o_in + r * DV + 4 * lane);
    float o[4] = {ov.x, ov.y, ov.z, ov.w}, zz[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) zz[j] = to_f32(zp[j]);
    const float4 wv = *reinterpret_cast<const float4 *>(w + 4 * lane);
    float ss = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
    const float rn = rsqrtf(ss / DV + eps);
    const float ww[4] = {wv.x, wv.y, wv.z, wv.w};
    if (live) {
#pragma unroll
        for (int j = 0; j < 4; ++j) op[j] = from_f32<OT>(o[j] * rn * ww[j] * silu(zz[j]));
    }
}

template <int DV, typename OT>
hipError_t norm_z(const Problem &p, const float *o, void *out, int64_t rows, hipStream_t s)
{
    constexpr int RPB = 256 / (DV / 4);
    const int64_t blocks = (rows + RPB - 1) / RPB;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (p.bf16)
        hipLaunchKernelGGL((gated_norm_kernel<DV, OT, bf16_t>), dim3((unsigned)blocks), dim3(256), 0, s,
                           o, static_cast<OT *>(out), static_cast<const bf16_t *>(p.z), p.norm_w, rows, p.eps);
    else
        hipLaunchKernelGGL((gated_norm_kernel<DV, OT, float>), dim3((unsigned)blocks), dim3(256), 0, s,
                           o, static_cast<OT *>(out), static_cast<const float *>(p.z), p.norm_w, rows, p.eps);
    return hipGetLastError();
}

template <int DV>
hipError_t norm_dv(const Problem &p, const float *o, void *out, int64_t rows, hipStream_t s)
{
    return p.out_bf16 ? norm_z<DV, bf16_t>(p, o, out, rows, s) : norm_z<DV, float>(p, o, out, rows, s);
}

}  // namespace

hipError_t launch_conv_state(const Problem &p, const void *qkv, const int32_t *cu, int single_T,
                             int32_t n_seqs, int64_t total_tokens, const float *conv_in,
                             float *conv_out, const int32_t *slot_in, const int32_t *slot_out,
                             hipStream_t s)
{
    const int cblocks = (p.conv_dim + 255) / 256;
    if ((int64_t)cblocks * n_seqs > 0x7fffffff) return hipErrorInvalidValue;
    dim3 grid(cblocks * n_seqs);
    if (p.bf16)
        hipLaunchKernelGGL((conv_state_kernel<bf16_t>), grid, dim3(256), 0, s,
                           static_cast<const bf16_t *>(qkv), total_tokens, p.conv_dim, conv_in, conv_out,
                           p.slot_stride, cu, single_T, slot_in, slot_out, cblocks);
    else
        hipLaunchKernelGGL((conv_state_kernel<float>), grid, dim3(256), 0, s,
                           static_cast<const float *>(qkv), total_tokens, p.conv_dim, conv_in, conv_out,
                           p.slot_stride, cu, single_T, slot_in, slot_out, cblocks);
    return hipGetLastError();
}

hipError_t launch_gated_norm(const Problem &p, const float *o, void *out, int64_t total_tokens, hipStream_t s)
{
    const int64_t rows = total_tokens * p.H_v;
    if (rows == 0) return hipSuccess;
    switch (p.d_v) {
    case 32: return norm_dv<32>(p, o, out, rows, s);
    case 64: return norm_dv<64>(p, o, out, rows, s);
    case 128: return norm_dv<128>(p, o, out, rows, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
