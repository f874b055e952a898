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
//
// Layer fusion (build_layer_attn_linear_core on the page "ik_llama.cpp
// src/llama-delta-net.cpp"), both optional and uniform per launch:
//   prologue: q, k, v are channel ranges of the mixed rows, each value the
//     silu of a 4-tap causal convolution over the channel's state and the
//     current row, formed as it is loaded;
//   epilogue: the workgroup holds a whole output row of its head, so the
//     gated RMSNorm o / sqrt(mean(o^2) + eps) * w * silu(z) is applied in
//     registers before the row is stored (one extra wave-level reduction).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kDecodeThreads = 256;

// Arguments of both recurrent kernels.
struct RecParams {
    const void *q, *k, *v;       // element type E; row strides rs_qk, rs_v
    const float *g, *beta;
    const float *state_in;       // recurrent state of slot 0 (null: zero states)
    float *state_out;
    void *out;
    const int32_t *cu, *slot_in, *slot_out;
    int T, H_k, H_v;
    int64_t slot_stride, rs_qk, rs_v;
    float scale, eps;
    Gates gates;
    const float *conv_w;         // [conv_dim][4]; null: no prologue
    const float *conv_in;        // slot rows (convolution state first); null: zero
    const void *z;               // [T][H_v][DV] gate, element type E; null: no epilogue
    const float *norm_w;         // [DV]
};

// Without raw gates the per-head parameters are never used, but they are
// still loaded (unconditional loads keep the compiler's count of outstanding
// memory operations exact): point them at g, which holds at least H_v values
// whenever a token exists.
Gates gates_of(const Problem &p, const float *g)
{
    return p.ssm_a ? Gates{p.ssm_a, p.ssm_dt, 1} : Gates{g, g, 0};
}

RecParams rec_params(const Problem &p, const void *q, const void *k, const void *v, const float *g,
                     const float *beta, const float *state_in, float *state_out, void *out,
                     const int32_t *cu, const int32_t *slot_in, const int32_t *slot_out, int T,
                     const float *conv_in)
{
    return RecParams{q, k, v, g, beta, state_in, state_out, out, cu, slot_in, slot_out, T,
                     p.H_k, p.H_v, p.slot_stride, p.rs_qk, p.rs_v, p.scale, p.eps, gates_of(p, g),
                     p.conv_w, conv_in, p.z, p.norm_w};
}

// One channel of the prologue: silu(w0 h0 + w1 h1 + w2 h2 + w3 x), with h the
// channel's three previous inputs (oldest first) and x the current one.
__device__ __forceinline__ float conv1(float4 w, float h0, float h1, float h2, float x)
{
    return silu(w.x * h0 + w.y * h1 + w.z * h2 + w.w * x);
}

// The three stored inputs of channel ch (zero without a state).
__device__ __forceinline__ void conv_hist(const RecParams &P, int sin, int64_t ch, float &h0, float &h1,
                                          float &h2)
{
    h0 = h1 = h2 = 0.f;
    if (sin >= 0) {
        const float *hp = P.conv_in + (int64_t)sin * P.slot_stride + ch * 3;
        h0 = hp[0];
        h1 = hp[1];
        h2 = hp[2];
    }
}

// Four consecutive channels from ch0 (a multiple of 4): 12 stored inputs.
__device__ __forceinline__ void conv_hist4(const RecParams &P, int sin, int64_t ch0, float hv[12])
{
#pragma unroll
    for (int j = 0; j < 12; ++j) hv[j] = 0.f;
    if (sin >= 0) {
        const float4 *hp = reinterpret_cast<const float4 *>(P.conv_in + (int64_t)sin * P.slot_stride + ch0 * 3);
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const float4 x = hp[j];
            hv[4 * j] = x.x; hv[4 * j + 1] = x.y; hv[4 * j + 2] = x.z; hv[4 * j + 3] = x.w;
        }
    }
}

// Gated RMSNorm of a row spread over CG consecutive lanes, four values each.
template <int CG, int DV>
__device__ __forceinline__ void gated_norm_row(float o[4], const float zz[4], const float nw[4], float eps)
{
    float ss = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
#pragma unroll
    for (int off = CG / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
    const float rn = rsqrtf(ss / DV + eps);
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = o[j] * rn * nw[j] * silu(zz[j]);
}

template <int DK, int DV, typename E, typename OT, bool FUSED>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(RecParams P)
{
    constexpr int CG = DV / 4;                  // float4 column groups
    constexpr int RG = kDecodeThreads / CG;     // row groups
    constexpr int RPT = DK / RG;                // state rows per thread
    static_assert(RPT >= 1 && RPT * RG == DK && 2 * DK <= kDecodeThreads, "bad decode tiling");

    const int i = blockIdx.x;                   // sequence (= token)
    const int h = blockIdx.y;                   // value head
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rg = tid / CG;
    const int col = cg * 4;
    const int kh = h / (P.H_v / P.H_k);         // blocked key-head sharing
    const E *q = static_cast<const E *>(P.q);
    const E *k = static_cast<const E *>(P.k);
    const E *v = static_cast<const E *>(P.v);
    const bool conv = FUSED && P.conv_w != nullptr;
    const bool norm = FUSED && P.z != nullptr;

    __shared__ float sk[DK];
    __shared__ float sq[DK];
    __shared__ float4 red[2][RG][CG];

    const int sin = P.state_in ? P.slot_in[i] : -1;
    const int sout = P.slot_out[i];

    // 1. stream the state block in (independent of everything else)
    float4 s[RPT];
    if (sin >= 0) {
        const float *base = P.state_in + (int64_t)sin * P.slot_stride + (int64_t)h * DK * DV + col;
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            s[r] = *reinterpret_cast<const float4 *>(base + (int64_t)(rg + r * RG) * DV);
    } else {
#pragma unroll
        for (int r = 0; r < RPT; ++r) s[r] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    // 2. q, k of the key head, v of this column group, scalars
    const int64_t qk_off = (int64_t)i * P.rs_qk + (int64_t)kh * DK;
    if (tid < 2 * DK) {
        const bool isk = tid < DK;
        const int e = isk ? tid : tid - DK;
        float x = to_f32((isk ? k : q)[qk_off + e]);
        if (conv) {
            const int64_t ch = (isk ? (int64_t)P.H_k * DK : 0) + (int64_t)kh * DK + e;
            float h0, h1, h2;
            conv_hist(P, sin, ch, h0, h1, h2);
            x = conv1(*reinterpret_cast<const float4 *>(P.conv_w + ch * 4), h0, h1, h2, x);
        }
        (isk ? sk : sq)[e] = x;
    }
    float gi = P.g[(int64_t)i * P.H_v + h];
    float bi = P.beta[(int64_t)i * P.H_v + h];
    {
        const float rate = P.gates.rate[h], bias = P.gates.bias[h];
        gi = P.gates.raw ? gate_g(gi, bias, rate) : gi;
        bi = P.gates.raw ? gate_beta(bi) : bi;
    }
    const E *vp = v + (int64_t)i * P.rs_v + (int64_t)h * DV + col;
    float vv[4] = {to_f32(vp[0]), to_f32(vp[1]), to_f32(vp[2]), to_f32(vp[3])};
    if (conv) {
        const int64_t ch0 = 2 * (int64_t)P.H_k * DK + (int64_t)h * DV + col;
        float hv[12];
        conv_hist4(P, sin, ch0, hv);
        const float4 *wp = reinterpret_cast<const float4 *>(P.conv_w + ch0 * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) vv[j] = conv1(wp[j], hv[3 * j], hv[3 * j + 1], hv[3 * j + 2], vv[j]);
    }
    float zz[4] = {0.f, 0.f, 0.f, 0.f}, nw[4] = {0.f, 0.f, 0.f, 0.f};
    if (norm) {
        const E *zp = static_cast<const E *>(P.z) + ((int64_t)i * P.H_v + h) * DV + col;
        const float4 w4 = *reinterpret_cast<const float4 *>(P.norm_w + col);
#pragma unroll
        for (int j = 0; j < 4; ++j) zz[j] = to_f32(zp[j]);
        nw[0] = w4.x; nw[1] = w4.y; nw[2] = w4.z; nw[3] = w4.w;
    }
    lds_sync();

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
    const float rk = rsqrtf(kk + P.eps);
    const float rq = rsqrtf(qq + P.eps) * P.scale;

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
    lds_sync();
    float4 tk = make_float4(0.f, 0.f, 0.f, 0.f), tq = tk;
#pragma unroll 8
    for (int j = 0; j < RG; ++j) {
        const float4 a = red[0][j][cg], b = red[1][j][cg];
        tk.x += a.x; tk.y += a.y; tk.z += a.z; tk.w += a.w;
        tq.x += b.x; tq.y += b.y; tq.z += b.z; tq.w += b.w;
    }

    // 5. delta rule and read-out (every row group holds its columns' row)
    const float dec = expf(gi);
    const float dk_ = dec * rk;
    float4 d;
    d.x = bi * (vv[0] - dk_ * tk.x);
    d.y = bi * (vv[1] - dk_ * tk.y);
    d.z = bi * (vv[2] - dk_ * tk.z);
    d.w = bi * (vv[3] - dk_ * tk.w);
    const float dq = dec * rq, kqh = rk * rq * kq;
    float o[4] = {dq * tq.x + kqh * d.x, dq * tq.y + kqh * d.y, dq * tq.z + kqh * d.z, dq * tq.w + kqh * d.w};
    if (norm) gated_norm_row<CG, DV>(o, zz, nw, P.eps);

    if (rg == 0) {
        OT *op = static_cast<OT *>(P.out) + ((int64_t)i * P.H_v + h) * DV + col;
#pragma unroll
        for (int j = 0; j < 4; ++j) op[j] = from_f32<OT>(o[j]);
    }

    // 6. rank-1 update of the decayed state and write-back
    if (sout >= 0) {
        float *base = P.state_out + (int64_t)sout * P.slot_stride + (int64_t)h * DK * DV + col;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const float kr = rk * sk[rg + r * RG];
            float4 u;
            u.x = dec * s[r].x + kr * d.x;
            u.y = dec * s[r].y + kr * d.y;
            u.z = dec * s[r].z + kr * d.z;
            u.w = dec * s[r].w + kr * d.w;
            *reinterpret_cast<float4 *>(base + (int64_t)(rg + r * RG) * DV) = u;
        }
    }
}

// Several tokens per sequence (speculative-decoding verification, short
// prompts): the same step, token after token, with the state block held in
// registers, so it is read from and written to HBM once per call instead of
// once per token.  q, k, v, g, beta (and z) of the next token are fetched
// while the current one is processed; k, q and the reduction partials
// alternate between two LDS buffers, so a token needs two barriers.  With the
// prologue, each thread keeps the convolution window of its channels in
// registers from token to token.  FUSED (here and in decode_kernel):
// prologue and/or epilogue present; the plain instantiation carries none of
// their code or registers.
// Sum over the row groups of one wave: lanes that hold the same column group
// (lane mod CG) and different row groups.
template <int CG>
__device__ __forceinline__ float rg_wave_sum(float x)
{
    if constexpr (CG <= 8) x += __shfl_xor(x, 8, 64);
    if constexpr (CG <= 16) x += __shfl_xor(x, 16, 64);
    // lanes l and l ^ 32 (v_permlane32_swap with both operands x: the low
    // half of the first result and the high half of the second hold x, the
    // other halves x of the partner lane).  The results pass through an
    // empty asm: with identical operands the compiler otherwise takes the
    // two results for one and adds the first to itself.
    const unsigned a = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(a, a, false, false);
    unsigned lo = r[0], hi = r[1];
    asm volatile("" : "+v"(lo), "+v"(hi));
    return __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
}

template <int DK, int DV, typename E, typename OT, bool FUSED>
__global__ __launch_bounds__(kDecodeThreads) void decode_multi_kernel(RecParams P)
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
    const int kh = h / (P.H_v / P.H_k);
    const int lane = tid & 63;
    const E *q = static_cast<const E *>(P.q);
    const E *k = static_cast<const E *>(P.k);
    const E *v = static_cast<const E *>(P.v);
    const bool conv = FUSED && P.conv_w != nullptr;
    const bool norm = FUSED && P.z != nullptr;

    __shared__ float sk[2][DK];
    __shared__ float sq[2][DK];
    constexpr int NW = kDecodeThreads / 64;
    __shared__ float4 red[2][2][NW][CG];

    // tokens of this sequence (clamped so that bad cu_seqlens stay in range)
    const int tb = min(max(P.cu[i], 0), P.T);
    const int te = min(max(P.cu[i + 1], tb), P.T);
    const int sin = P.state_in ? P.slot_in[i] : -1;
    const int sout = P.slot_out[i];

    float4 s[RPT];
    if (sin >= 0) {
        const float *base = P.state_in + (int64_t)sin * P.slot_stride + (int64_t)h * DK * DV + col;
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            s[r] = *reinterpret_cast<const float4 *>(base + (int64_t)(rg + r * RG) * DV);
    } else {
#pragma unroll
        for (int r = 0; r < RPT; ++r) s[r] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    // prologue: taps and stored inputs of this thread's k or q channel and of
    // its four v channels
    const bool isk = tid < DK;
    const int64_t chq = (isk ? (int64_t)P.H_k * DK : 0) + (int64_t)kh * DK + (isk ? tid : tid - DK);
    const int64_t chv = 2 * (int64_t)P.H_k * DK + (int64_t)h * DV + col;
    float4 wq = make_float4(0.f, 0.f, 0.f, 0.f), wv[4];
    float hq[3] = {0.f, 0.f, 0.f}, hv[12];
#pragma unroll
    for (int j = 0; j < 4; ++j) wv[j] = wq;
#pragma unroll
    for (int j = 0; j < 12; ++j) hv[j] = 0.f;
    if (conv) {
        if (tid < 2 * DK) {
            wq = *reinterpret_cast<const float4 *>(P.conv_w + chq * 4);
            conv_hist(P, sin, chq, hq[0], hq[1], hq[2]);
        }
        const float4 *wp = reinterpret_cast<const float4 *>(P.conv_w + chv * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) wv[j] = wp[j];
        conv_hist4(P, sin, chv, hv);
    }
    float nw[4] = {0.f, 0.f, 0.f, 0.f};
    if (norm) {
        const float4 w4 = *reinterpret_cast<const float4 *>(P.norm_w + col);
        nw[0] = w4.x; nw[1] = w4.y; nw[2] = w4.z; nw[3] = w4.w;
    }

    // this thread's share of a token: one of k (tid < DK) or q (DK <= tid <
    // 2 DK), four values of v (and of z), and the token's g and beta
    struct Tok {
        float kq, gt, bt;
        float vv[4], zz[4];
    };
    auto fetch = [&](int t) {
        Tok r;
        const int64_t qk_off = (int64_t)t * P.rs_qk + (int64_t)kh * DK;
        r.kq = tid < DK ? to_f32(k[qk_off + tid]) : tid < 2 * DK ? to_f32(q[qk_off + tid - DK]) : 0.f;
        r.gt = P.g[(int64_t)t * P.H_v + h];
        r.bt = P.beta[(int64_t)t * P.H_v + h];
        const float rate = P.gates.rate[h], bias = P.gates.bias[h];
        r.gt = P.gates.raw ? gate_g(r.gt, bias, rate) : r.gt;
        r.bt = P.gates.raw ? gate_beta(r.bt) : r.bt;
        const E *vp = v + (int64_t)t * P.rs_v + (int64_t)h * DV + col;
#pragma unroll
        for (int j = 0; j < 4; ++j) r.vv[j] = to_f32(vp[j]);
        // z (read from v, same layout, when there is no epilogue: an
        // unconditional load keeps the compiler's count of loads exact)
        if constexpr (FUSED) {
            const E *zp = norm ? static_cast<const E *>(P.z) + ((int64_t)t * P.H_v + h) * DV + col
                               : v + (int64_t)t * P.rs_v + (int64_t)h * DV + col;
#pragma unroll
            for (int j = 0; j < 4; ++j) r.zz[j] = to_f32(zp[j]);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) r.zz[j] = 0.f;
        }
        return r;
    };
    Tok cur{};
    if (tb < te) cur = fetch(tb);               // an empty sequence reads no token

    for (int t = tb; t < te; ++t) {
        const int b = (t - tb) & 1;
        float kqv = cur.kq;
        float vv[4] = {cur.vv[0], cur.vv[1], cur.vv[2], cur.vv[3]};
        if (conv) {
            kqv = conv1(wq, hq[0], hq[1], hq[2], cur.kq);
            hq[0] = hq[1]; hq[1] = hq[2]; hq[2] = cur.kq;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                vv[j] = conv1(wv[j], hv[3 * j], hv[3 * j + 1], hv[3 * j + 2], cur.vv[j]);
                hv[3 * j] = hv[3 * j + 1]; hv[3 * j + 1] = hv[3 * j + 2]; hv[3 * j + 2] = cur.vv[j];
            }
        }
        if (tid < DK) sk[b][tid] = kqv;
        else if (tid < 2 * DK) sq[b][tid - DK] = kqv;
        const Tok nxt = fetch(min(t + 1, te - 1));
        lds_sync();

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
        const float rk = rsqrtf(kk + P.eps);
        const float rq = rsqrtf(qq + P.eps) * P.scale;

        // partial column reductions of the state before this token
        float4 pk = make_float4(0.f, 0.f, 0.f, 0.f), pq = pk;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const float a = sk[b][rg + r * RG], c = sq[b][rg + r * RG];
            pk.x += s[r].x * a; pk.y += s[r].y * a; pk.z += s[r].z * a; pk.w += s[r].w * a;
            pq.x += s[r].x * c; pq.y += s[r].y * c; pq.z += s[r].z * c; pq.w += s[r].w * c;
        }
        // the wave's row groups first (lane exchanges), then the waves (LDS)
        pk.x = rg_wave_sum<CG>(pk.x); pk.y = rg_wave_sum<CG>(pk.y); pk.z = rg_wave_sum<CG>(pk.z); pk.w = rg_wave_sum<CG>(pk.w);
        pq.x = rg_wave_sum<CG>(pq.x); pq.y = rg_wave_sum<CG>(pq.y); pq.z = rg_wave_sum<CG>(pq.z); pq.w = rg_wave_sum<CG>(pq.w);
        if (lane < CG) {
            red[b][0][tid >> 6][cg] = pk;
            red[b][1][tid >> 6][cg] = pq;
        }
        lds_sync();
        float4 tk = make_float4(0.f, 0.f, 0.f, 0.f), tq = tk;
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            const float4 a = red[b][0][j][cg], c = red[b][1][j][cg];
            tk.x += a.x; tk.y += a.y; tk.z += a.z; tk.w += a.w;
            tq.x += c.x; tq.y += c.y; tq.z += c.z; tq.w += c.w;
        }

        // delta rule and read-out
        const float dec = expf(cur.gt);
        const float dk_ = dec * rk;
        float4 d;
        d.x = cur.bt * (vv[0] - dk_ * tk.x);
        d.y = cur.bt * (vv[1] - dk_ * tk.y);
        d.z = cur.bt * (vv[2] - dk_ * tk.z);
        d.w = cur.bt * (vv[3] - dk_ * tk.w);
        const float dq = dec * rq, kqh = rk * rq * kq;
        float o[4] = {dq * tq.x + kqh * d.x, dq * tq.y + kqh * d.y, dq * tq.z + kqh * d.z,
                      dq * tq.w + kqh * d.w};
        if (norm) gated_norm_row<CG, DV>(o, cur.zz, nw, P.eps);
        {
            // row group 0 writes the row; the other lanes' offsets fall past
            // the buffer's end and are dropped.  No branch: a store inside one
            // would make the next wait for the prefetched token wait for it
            // too (on gfx9 stores and loads share the counter).
            const __amdgpu_buffer_rsrc_t ob =
                raw_buffer(static_cast<OT *>(P.out) + ((int64_t)t * P.H_v + h) * DV, (uint32_t)(DV * sizeof(OT)));
            const uint32_t off = rg == 0 ? (uint32_t)(col * sizeof(OT)) : 0x80000000u;
#pragma unroll
            for (int j = 0; j < 4; ++j) buffer_store(from_f32<OT>(o[j]), ob, off + (uint32_t)(j * sizeof(OT)));
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
        float *base = P.state_out + (int64_t)sout * P.slot_stride + (int64_t)h * DK * DV + col;
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            *reinterpret_cast<float4 *>(base + (int64_t)(rg + r * RG) * DV) = s[r];
    }
}

template <int DK, int DV, typename E, typename OT>
hipError_t launch_multi_t(const Problem &p, const DecodeMultiArgs &a, hipStream_t st)
{
    const RecParams P = rec_params(p, a.q, a.k, a.v, a.g, a.beta, a.state_in, a.state_out, a.out,
                                   a.cu_seqlens, a.slot_in, a.slot_out, (int)a.total_tokens, a.conv_in);
    if (p.conv_w || p.z)
        hipLaunchKernelGGL((decode_multi_kernel<DK, DV, E, OT, true>), dim3(a.n_seqs, p.H_v),
                           dim3(kDecodeThreads), 0, st, P);
    else
        hipLaunchKernelGGL((decode_multi_kernel<DK, DV, E, OT, false>), dim3(a.n_seqs, p.H_v),
                           dim3(kDecodeThreads), 0, st, P);
    return hipGetLastError();
}

template <int DK, int DV, typename E, typename OT>
hipError_t launch_t(const Problem &p, const DecodeArgs &a, hipStream_t st)
{
    const RecParams P = rec_params(p, a.q, a.k, a.v, a.g, a.beta, a.state_in, a.state_out, a.out,
                                   nullptr, a.slot_in, a.slot_out, a.n_seqs, a.conv_in);
    if (p.conv_w || p.z)
        hipLaunchKernelGGL((decode_kernel<DK, DV, E, OT, true>), dim3(a.n_seqs, p.H_v), dim3(kDecodeThreads), 0,
                           st, P);
    else
        hipLaunchKernelGGL((decode_kernel<DK, DV, E, OT, false>), dim3(a.n_seqs, p.H_v), dim3(kDecodeThreads), 0,
                           st, P);
    return hipGetLastError();
}

template <int DK, int DV, typename Args, bool MULTI>
hipError_t launch_types(const Problem &p, const Args &a, hipStream_t st)
{
    if constexpr (MULTI) {
        if (p.bf16)
            return p.out_bf16 ? launch_multi_t<DK, DV, bf16_t, bf16_t>(p, a, st)
                              : launch_multi_t<DK, DV, bf16_t, float>(p, a, st);
        return p.out_bf16 ? launch_multi_t<DK, DV, float, bf16_t>(p, a, st)
                          : launch_multi_t<DK, DV, float, float>(p, a, st);
    } else {
        if (p.bf16)
            return p.out_bf16 ? launch_t<DK, DV, bf16_t, bf16_t>(p, a, st) : launch_t<DK, DV, bf16_t, float>(p, a, st);
        return p.out_bf16 ? launch_t<DK, DV, float, bf16_t>(p, a, st) : launch_t<DK, DV, float, float>(p, a, st);
    }
}

template <int DK, typename Args, bool MULTI>
hipError_t launch_dk(const Problem &p, const Args &a, hipStream_t st)
{
    switch (p.d_v) {
    case 32: return launch_types<DK, 32, Args, MULTI>(p, a, st);
    case 64: return launch_types<DK, 64, Args, MULTI>(p, a, st);
    case 128: return launch_types<DK, 128, Args, MULTI>(p, a, st);
    }
    return hipErrorInvalidValue;
}

template <typename Args, bool MULTI>
hipError_t launch_any(const Problem &p, const Args &a, hipStream_t st)
{
    switch (p.d_k) {
    case 32: return launch_dk<32, Args, MULTI>(p, a, st);
    case 64: return launch_dk<64, Args, MULTI>(p, a, st);
    case 128: return launch_dk<128, Args, MULTI>(p, a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const Problem &p, const DecodeArgs &a, hipStream_t st)
{
    return launch_any<DecodeArgs, false>(p, a, st);
}

hipError_t launch_decode_multi(const Problem &p, const DecodeMultiArgs &a, hipStream_t st)
{
    return launch_any<DecodeMultiArgs, true>(p, a, st);
}

}  // namespace gdn
