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

// Without raw gates the per-head parameters are never used, but they are
// still loaded (unconditional loads keep the compiler's count of outstanding
// memory operations exact): point them at g, which holds at least H_v values
// whenever a token exists.
Gates gates_of(const Problem &p, const float *g)
{
    return p.ssm_a ? Gates{p.ssm_a, p.ssm_dt, 1} : Gates{g, g, 0};
}

template <int DK, int DV, int DVB, typename E, typename OT>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const float *state_in, float *state_out, OT *__restrict__ out,
    const int32_t *__restrict__ slot_in, const int32_t *__restrict__ slot_out,
    int H_k, int H_v, int64_t slot_stride, float scale, float eps, Gates gates)
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
    float gi = g[(int64_t)i * H_v + h];
    float bi = beta[(int64_t)i * H_v + h];
    {
        const float rate = gates.rate[h], bias = gates.bias[h];
        gi = gates.raw ? gate_g(gi, bias, rate) : gi;
        bi = gates.raw ? gate_beta(bi) : bi;
    }
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

// Several tokens per sequence (speculative-decoding verification, short
// prompts): the same step, token after token, with the state block held in
// registers, so it is read from and written to HBM once per call instead of
// once per token.  q, k, v, g, beta of the next token are fetched while the
// current one is processed; k, q and the reduction partials alternate between
// two LDS buffers, so a token needs two barriers.
template <int DK, int DV, typename E, typename OT>
__global__ __launch_bounds__(kDecodeThreads) void decode_multi_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const float *state_in, float *state_out, OT *__restrict__ out,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ slot_in,
    const int32_t *__restrict__ slot_out, int T, int H_k, int H_v, int64_t slot_stride,
    float scale, float eps, Gates gates)
{
    constexpr int CG = DV / 4;                  // float4 column groups
    constexpr int RG = kDecodeThreads / CG;     // row groups
    constexpr int RPT = DK / RG;                // state rows per thread
    static_assert(RPT >= 1 && RPT * RG == DK && 2 * DK <= kDecodeThreads, "bad decode tiling");

    const int i = blockIdx.x;                   // sequence
    const int h = blockIdx.y;                   // value head
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rg = tid / CG;
    const int col = cg * 4;
    const int kh = h / (H_v / H_k);
    const int lane = tid & 63;

    __shared__ float sk[2][DK];
    __shared__ float sq[2][DK];
    __shared__ float4 red[2][2][RG][CG];

    // tokens of this sequence (clamped so that bad cu_seqlens stay in range)
    const int tb = min(max(cu[i], 0), T);
    const int te = min(max(cu[i + 1], tb), T);
    const int sin = state_in ? slot_in[i] : -1;
    const int sout = slot_out[i];

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

    // this thread's share of a token: one of k (tid < DK) or q (DK <= tid <
    // 2 DK), four values of v, and the token's g and beta
    struct Tok {
        float kq, gt, bt;
        float vv[4];
    };
    auto fetch = [&](int t) {
        Tok r;
        const int64_t qk_off = ((int64_t)t * H_k + kh) * DK;
        r.kq = tid < DK ? to_f32(k[qk_off + tid]) : tid < 2 * DK ? to_f32(q[qk_off + tid - DK]) : 0.f;
        r.gt = g[(int64_t)t * H_v + h];
        r.bt = beta[(int64_t)t * H_v + h];
        const float rate = gates.rate[h], bias = gates.bias[h];
        r.gt = gates.raw ? gate_g(r.gt, bias, rate) : r.gt;
        r.bt = gates.raw ? gate_beta(r.bt) : r.bt;
        const E *vp = v + ((int64_t)t * H_v + h) * DV + col;
#pragma unroll
        for (int j = 0; j < 4; ++j) r.vv[j] = to_f32(vp[j]);
        return r;
    };
    Tok cur{};
    if (tb < te) cur = fetch(tb);               // an empty sequence reads no token

    for (int t = tb; t < te; ++t) {
        const int b = (t - tb) & 1;
        if (tid < DK) sk[b][tid] = cur.kq;
        else if (tid < 2 * DK) sq[b][tid - DK] = cur.kq;
        const Tok nxt = fetch(min(t + 1, te - 1));
        __syncthreads();

        // norms (every wave reduces redundantly; no extra barrier)
        float kk = 0.f, qq = 0.f, kq = 0.f;
        for (int j = lane; j < DK; j += 64) {
            const float a = sk[b][j], c = sq[b][j];
            kk += a * a;
            qq += c * c;
            kq += a * c;
        }
        kk = wave_sum(kk);
        qq = wave_sum(qq);
        kq = wave_sum(kq);
        const float rk = rsqrtf(kk + eps);
        const float rq = rsqrtf(qq + eps) * scale;

        // partial column reductions of the state before this token
        float4 pk = make_float4(0.f, 0.f, 0.f, 0.f), pq = pk;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const float a = sk[b][rg + r * RG], c = sq[b][rg + r * RG];
            pk.x += s[r].x * a; pk.y += s[r].y * a; pk.z += s[r].z * a; pk.w += s[r].w * a;
            pq.x += s[r].x * c; pq.y += s[r].y * c; pq.z += s[r].z * c; pq.w += s[r].w * c;
        }
        red[b][0][rg][cg] = pk;
        red[b][1][rg][cg] = pq;
        __syncthreads();
        float4 tk = make_float4(0.f, 0.f, 0.f, 0.f), tq = tk;
#pragma unroll 8
        for (int j = 0; j < RG; ++j) {
            const float4 a = red[b][0][j][cg], c = red[b][1][j][cg];
            tk.x += a.x; tk.y += a.y; tk.z += a.z; tk.w += a.w;
            tq.x += c.x; tq.y += c.y; tq.z += c.z; tq.w += c.w;
        }

        // delta rule and read-out
        const float dec = expf(cur.gt);
        const float dk_ = dec * rk;
        float4 d;
        d.x = cur.bt * (cur.vv[0] - dk_ * tk.x);
        d.y = cur.bt * (cur.vv[1] - dk_ * tk.y);
        d.z = cur.bt * (cur.vv[2] - dk_ * tk.z);
        d.w = cur.bt * (cur.vv[3] - dk_ * tk.w);
        const float dq = dec * rq, kqh = rk * rq * kq;
        if (rg == 0) {
            OT *op = out + ((int64_t)t * H_v + h) * DV + col;
            op[0] = from_f32<OT>(dq * tq.x + kqh * d.x);
            op[1] = from_f32<OT>(dq * tq.y + kqh * d.y);
            op[2] = from_f32<OT>(dq * tq.z + kqh * d.z);
            op[3] = from_f32<OT>(dq * tq.w + kqh * d.w);
        }
        // rank-1 update of the decayed state, in registers
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const float kr = rk * sk[b][rg + r * RG];
            s[r].x = dec * s[r].x + kr * d.x;
            s[r].y = dec * s[r].y + kr * d.y;
            s[r].z = dec * s[r].z + kr * d.z;
            s[r].w = dec * s[r].w + kr * d.w;
        }
        cur = nxt;
    }

    if (sout >= 0) {
        float *base = state_out + (int64_t)sout * slot_stride + (int64_t)h * DK * DV + col;
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            *reinterpret_cast<float4 *>(base + (int64_t)(rg + r * RG) * DV) = s[r];
    }
}

template <int DK, int DV, typename E, typename OT>
hipError_t launch_multi_t(const Problem &p, const DecodeMultiArgs &a, hipStream_t st)
{
    hipLaunchKernelGGL((decode_multi_kernel<DK, DV, E, OT>), dim3(a.n_seqs, p.H_v), dim3(kDecodeThreads), 0,
                       st, static_cast<const E *>(a.q), static_cast<const E *>(a.k),
                       static_cast<const E *>(a.v), a.g, a.beta, a.state_in, a.state_out,
                       static_cast<OT *>(a.out), a.cu_seqlens, a.slot_in, a.slot_out,
                       (int)a.total_tokens, p.H_k, p.H_v, p.slot_stride, p.scale, p.eps,
                       gates_of(p, a.g));
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_multi_dv(const Problem &p, const DecodeMultiArgs &a, hipStream_t st)
{
    if (p.bf16)
        return p.out_bf16 ? launch_multi_t<DK, DV, bf16_t, bf16_t>(p, a, st)
                          : launch_multi_t<DK, DV, bf16_t, float>(p, a, st);
    return p.out_bf16 ? launch_multi_t<DK, DV, float, bf16_t>(p, a, st) : launch_multi_t<DK, DV, float, float>(p, a, st);
}

template <int DK>
hipError_t launch_multi_dk(const Problem &p, const DecodeMultiArgs &a, hipStream_t st)
{
    switch (p.d_v) {
    case 32: return launch_multi_dv<DK, 32>(p, a, st);
    case 64: return launch_multi_dv<DK, 64>(p, a, st);
    case 128: return launch_multi_dv<DK, 128>(p, a, st);
    }
    return hipErrorInvalidValue;
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
                       p.slot_stride, p.scale, p.eps, gates_of(p, a.g));
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

hipError_t launch_decode_multi(const Problem &p, const DecodeMultiArgs &a, hipStream_t st)
{
    switch (p.d_k) {
    case 32: return launch_multi_dk<32>(p, a, st);
    case 64: return launch_multi_dk<64>(p, a, st);
    case 128: return launch_multi_dk<128>(p, a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
