// gdn_decode.hip -- autoregressive step of the gated delta rule (one token per
// sequence), the graph build_delta_net_autoregressive of the page
// "Optimization: Qwen3 next autoregressive pass (#17996)":
//
//   S' = exp(g) S;  kv = S'^T k^;  delta = beta (v - kv);  S = S' + k^ (x) delta;
//   o = S^T q^ = exp(g) (S_old^T q^) + (k^ . q^) delta
//
// Work is HBM-bound (0.875 flop per state byte), so no matrix cores: one
// workgroup owns a d_k x DVB column block of one (sequence, value head) state,
// streams it from HBM once with 16-byte coalesced loads, forms both column
// reductions S^T k and S^T q from the same registers (partials combined
// through LDS), and writes the updated block back once.  The two reductions
// use the OLD state; the decay is applied to the reduced vectors, which is
// the same arithmetic reordered.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kDecodeThreads = 256;

template <int DK, int DV, int DVB, typename E, typename OT>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const float *state_in, float *state_out, OT *__restrict__ out,
    const int32_t *__restrict__ slot_in, const int32_t *__restrict__ slot_out,
    int H_k, int H_v, int64_t slot_stride, float scale, float eps)
{
    constexpr int CG = DVB / 4;                 // float4 column groups
    constexpr int RG = kDecodeThreads / CG;     // row groups
    constexpr int RPT = DK / RG;                // state rows per thread
    static_assert(RPT >= 1 && RPT * RG == DK, "bad decode tiling");

    const int i = blockIdx.x;                   // sequence (= token)
    const int h = blockIdx.y;                   // value head
    const int col0 = blockIdx.z * DVB;
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rg = tid / CG;
    const int col = col0 + cg * 4;
    const int kh = h / (H_v / H_k);             // blocked key-head sharing

    __shared__ float sk[DK];
    __shared__ float sq[DK];
    __shared__ float4 red[2][RG][CG];

    const int sin = state_in ? slot_in[i] : -1;
    const int sout = slot_out[i];

    // 1. stream the state block in (independent of everything else)
    float4 s[RPT];
    if (sin >= 0) {
        const float *base = state_in + (int64_t)sin * slot_stride + (int64_t)h * DK * DV + col;
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            s[r] = *reinterpret_cast<const float4 *>(base + (int64_t)(rg + r * RG) * DV);
    } else {
#pragma unroll
        for (int r = 0; r < RPT; ++r) s[r] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    // 2. q, k of the key head, v of this column group, scalars
    const int64_t qk_off = ((int64_t)i * H_k + kh) * DK;
    if (tid < DK) sk[tid] = to_f32(k[qk_off + tid]);
    else if (tid < 2 * DK) sq[tid - DK] = to_f32(q[qk_off + tid - DK]);
    const float gi = g[(int64_t)i * H_v + h];
    const float bi = beta[(int64_t)i * H_v + h];
    const E *vp = v + ((int64_t)i * H_v + h) * DV + col;
    const float v0 = to_f32(vp[0]), v1 = to_f32(vp[1]), v2 = to_f32(vp[2]), v3 = to_f32(vp[3]);
    __syncthreads();

    // 3. norms (every wave reduces redundantly; no extra barrier)
    float kk = 0.f, qq = 0.f, kq = 0.f;
    const int lane = tid & 63;
    for (int j = lane; j < DK; j += 64) {
        const float a = sk[j], b = sq[j];
        kk += a * a;
        qq += b * b;
        kq += a * b;
    }
    kk = wave_sum(kk);
    qq = wave_sum(qq);
    kq = wave_sum(kq);
    const float rk = rsqrtf(kk + eps);
    const float rq = rsqrtf(qq + eps) * scale;

    // 4. partial column reductions of the old state: sum_r S[r][c] k[r], q[r]
    float4 pk = make_float4(0.f, 0.f, 0.f, 0.f), pq = pk;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const float a = sk[rg + r * RG], b = sq[rg + r * RG];
        pk.x += s[r].x * a; pk.y += s[r].y * a; pk.z += s[r].z * a; pk.w += s[r].w * a;
        pq.x += s[r].x * b; pq.y += s[r].y * b; pq.z += s[r].z * b; pq.w += s[r].w * b;
    }
    red[0][rg][cg] = pk;
    red[1][rg][cg] = pq;
    __syncthreads();
    float4 tk = make_float4(0.f, 0.f, 0.f, 0.f), tq = tk;
#pragma unroll 8
    for (int j = 0; j < RG; ++j) {
        const float4 a = red[0][j][cg], b = red[1][j][cg];
        tk.x += a.x; tk.y += a.y; tk.z += a.z; tk.w += a.w;
        tq.x += b.x; tq.y += b.y; tq.z += b.z; tq.w += b.w;
    }

    // 5. delta rule and read-out
    const float dec = expf(gi);
    const float dk_ = dec * rk;
    float4 d;
    d.x = bi * (v0 - dk_ * tk.x);
    d.y = bi * (v1 - dk_ * tk.y);
    d.z = bi * (v2 - dk_ * tk.z);
    d.w = bi * (v3 - dk_ * tk.w);
    const float dq = dec * rq, kqh = rk * rq * kq;

    if (rg == 0) {
        OT *op = out + ((int64_t)i * H_v + h) * DV + col;
        op[0] = from_f32<OT>(dq * tq.x + kqh * d.x);
        op[1] = from_f32<OT>(dq * tq.y + kqh * d.y);
        op[2] = from_f32<OT>(dq * tq.z + kqh * d.z);
        op[3] = from_f32<OT>(dq * tq.w + kqh * d.w);
    }

    // 6. rank-1 update of the decayed state and write-back
    if (sout >= 0) {
        float *base = state_out + (int64_t)sout * slot_stride + (int64_t)h * DK * DV + col;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const float kr = rk * sk[rg + r * RG];
            float4 o;
            o.x = dec * s[r].x + kr * d.x;
            o.y = dec * s[r].y + kr * d.y;
            o.z = dec * s[r].z + kr * d.z;
            o.w = dec * s[r].w + kr * d.w;
            *reinterpret_cast<float4 *>(base + (int64_t)(rg + r * RG) * DV) = o;
        }
    }
}

template <int DK, int DV, typename E, typename OT>
hipError_t launch_t(const Problem &p, const DecodeArgs &a, hipStream_t st)
{
    constexpr int DVB = DV;     // one workgroup per (sequence, head)
    dim3 grid(a.n_seqs, p.H_v, DV / DVB);
    hipLaunchKernelGGL((decode_kernel<DK, DV, DVB, E, OT>), grid, dim3(kDecodeThreads), 0, st,
                       static_cast<const E *>(a.q), static_cast<const E *>(a.k),
                       static_cast<const E *>(a.v), a.g, a.beta, a.state_in, a.state_out,
                       static_cast<OT *>(a.out), a.slot_in, a.slot_out, p.H_k, p.H_v,
                       p.slot_stride, p.scale, p.eps);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_dv(const Problem &p, const DecodeArgs &a, hipStream_t st)
{
    if (p.bf16)
        return p.out_bf16 ? launch_t<DK, DV, bf16_t, bf16_t>(p, a, st) : launch_t<DK, DV, bf16_t, float>(p, a, st);
    return p.out_bf16 ? launch_t<DK, DV, float, bf16_t>(p, a, st) : launch_t<DK, DV, float, float>(p, a, st);
}

template <int DK>
hipError_t launch_dk(const Problem &p, const DecodeArgs &a, hipStream_t st)
{
    switch (p.d_v) {
    case 32: return launch_dv<DK, 32>(p, a, st);
    case 64: return launch_dv<DK, 64>(p, a, st);
    case 128: return launch_dv<DK, 128>(p, a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const Problem &p, const DecodeArgs &a, hipStream_t st)
{
    switch (p.d_k) {
    case 32: return launch_dk<32>(p, a, st);
    case 64: return launch_dk<64>(p, a, st);
    case 128: return launch_dk<128>(p, a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
