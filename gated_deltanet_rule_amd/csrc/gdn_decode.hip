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
// With the prologue and H_v / H_k = 1 or 2, a workgroup takes every value
// head of one key head (GR = H_v / H_k groups of 256 threads, one value head
// each): it is then the only reader of the convolution state of the key
// head's q and k channels and of its value heads' v channels, and replaces
// that state (the last three inputs of each channel) itself, in place, once
// every thread has read the old values.  Other head ratios keep one value
// head per workgroup and leave the state to conv_state_kernel.
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
    float *conv_out;             // slot rows receiving the new convolution state
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
                     const float *conv_in, float *conv_out)
{
    return RecParams{q, k, v, g, beta, state_in, state_out, out, cu, slot_in, slot_out, T,
                     p.H_k, p.H_v, p.slot_stride, p.rs_qk, p.rs_v, p.scale, p.eps, gates_of(p, g),
                     p.conv_w, conv_in, conv_out, p.z, p.norm_w};
}


// One channel of the prologue: silu(w0 h0 + w1 h1 + w2 h2 + w3 x), with h the
// channel's three previous inputs (oldest first) and x the current one.
__device__ __forceinline__ float conv1(float4 w, float h0, float h1, float h2, float x)
{
    return silu(w.x * h0 + w.y * h1 + w.z * h2 + w.w * x);
}

// Gated RMSNorm of a row spread over CG consecutive lanes, four values each;
// zg = w * silu(z) of the same four columns.
template <int CG, int DV>
__device__ __forceinline__ void gated_norm_row(float o[4], const float zg[4], float eps)
{
    const float ss = group_sum<CG>(o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3]);
    const float rn = rsqrtf(ss / DV + eps);
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = o[j] * rn * zg[j];
}

// Four consecutive values of E through a buffer resource (one 8- or
// 16-byte access; zeros past the range's end).
template <typename E> __device__ __forceinline__ void buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off, float f[4]);
template <> __device__ __forceinline__ void buf_load4<bf16_t>(__amdgpu_buffer_rsrc_t r, uint32_t off, float f[4]) {
    const u32x2 u = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    f[0] = __uint_as_float(u.x << 16);
    f[1] = __uint_as_float(u.x & 0xffff0000u);
    f[2] = __uint_as_float(u.y << 16);
    f[3] = __uint_as_float(u.y & 0xffff0000u);
}
template <> __device__ __forceinline__ void buf_load4<float>(__amdgpu_buffer_rsrc_t r, uint32_t off, float f[4]) {
    const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
}
__device__ __forceinline__ float4 buf_load_f4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
    const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
    return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
}
// The loads that produced v are complete at this point of the program (the
// compiler's wait for them is placed here); no code is emitted.
__device__ __forceinline__ void loaded(float v) { asm volatile("" ::"v"(v)); }

// GR > 1 only with the prologue: GR value heads (those of key head
// blockIdx.y), one per group of kDecodeThreads threads.
//
// Order of memory operations: every small input (q, k, v, the gates and,
// when fused, the convolution taps and state, z and the norm weight) is
// loaded before the state block, and none of these loads sits behind a
// branch.  The wait counter completes loads in issue order, so the prologue's
// wait for them leaves the state block's loads in flight: the prologue, the
// norms of q and k and their exchange through LDS overlap the stream of the
// state, instead of each following it as a further round trip.  Inputs that
// may be absent (a state slot of -1, no state pool, a part of the fusion
// switched off) are read through empty buffer ranges, which return zeros
// without touching memory.
template <int DK, int DV, typename E, typename OT, bool FUSED, int GR>
__global__ __launch_bounds__(kDecodeThreads * GR, 4) void decode_kernel(RecParams P)
{
    constexpr int CG = DV / 4;                  // float4 column groups
    constexpr int RG = kDecodeThreads / CG;     // row groups
    constexpr int RPT = DK / RG;                // state rows per thread
    static_assert(RPT >= 1 && RPT * RG == DK && 2 * DK <= kDecodeThreads, "bad decode tiling");

    const int i = blockIdx.x;                   // sequence (= token)
    const int grp = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kDecodeThreads);
    const int tid = (int)threadIdx.x % kDecodeThreads;
    const int cg = tid % CG;
    const int rg = tid / CG;
    const int col = cg * 4;
    const int h = GR > 1 ? (int)blockIdx.y * GR + grp : (int)blockIdx.y;   // value head
    const int kh = h / (P.H_v / P.H_k);         // blocked key-head sharing
    const E *q = static_cast<const E *>(P.q);
    const E *k = static_cast<const E *>(P.k);
    const E *v = static_cast<const E *>(P.v);
    const bool conv = FUSED && P.conv_w != nullptr;
    const bool norm = FUSED && P.z != nullptr;

    __shared__ float sk_[GR][DK];
    __shared__ float sq_[GR][DK];
    __shared__ float4 red_[GR][2][RG][CG];
    // fused: v after the prologue and w * silu(z), one value per channel
    __shared__ __attribute__((aligned(16))) float sv_[FUSED ? GR : 1][FUSED ? DV : 1];
    __shared__ __attribute__((aligned(16))) float sz_[FUSED ? GR : 1][FUSED ? DV : 1];
    float *sk = sk_[grp];
    float *sq = sq_[grp];
    float4(&red)[2][RG][CG] = red_[grp];

    const int sin = P.state_in ? P.slot_in[i] : -1;
    const int sout = P.slot_out[i];

    // 1. small inputs: one q or k channel of the key head per thread (the
    //    threads past 2 DK repeat one), the scalars, and v: four columns per
    //    thread, or (fused) one channel per thread, whose convolution and
    //    norm gate are formed once and shared through LDS
    const int e2 = tid % (2 * DK);
    const bool isk = e2 < DK;
    const int e = isk ? e2 : e2 - DK;
    const int ev = tid % DV;
    float x = to_f32((isk ? k : q)[(int64_t)i * P.rs_qk + (int64_t)kh * DK + e]);
    const E *vrow = v + (int64_t)i * P.rs_v + (int64_t)h * DV;
    float vv[4];
    float xv = 0.f;
    if constexpr (FUSED)
        xv = to_f32(vrow[ev]);
    else
        buf_load4<E>(raw_buffer(const_cast<E *>(vrow), DV * sizeof(E)), col * sizeof(E), vv);
    float gi = P.g[(int64_t)i * P.H_v + h];
    float bi = P.beta[(int64_t)i * P.H_v + h];
    const float rate = P.gates.rate[h], bias = P.gates.bias[h];
    // prologue and epilogue inputs: taps and stored inputs of this thread's q
    // or k channel and v channel, its z and norm weight
    const int conv_dim = 2 * P.H_k * DK + P.H_v * DV;
    const int64_t ch = (isk ? (int64_t)P.H_k * DK : 0) + (int64_t)kh * DK + e;
    const int64_t chv = 2 * (int64_t)P.H_k * DK + (int64_t)h * DV + ev;
    u32x3 hq = {0u, 0u, 0u}, hv = {0u, 0u, 0u};
    float4 wq = make_float4(0.f, 0.f, 0.f, 0.f), wv = wq;
    float zs = 0.f, nws = 0.f;
    if constexpr (FUSED) {
        const bool hist = conv && sin >= 0;
        const auto hb = raw_buffer(hist ? const_cast<float *>(P.conv_in + (int64_t)sin * P.slot_stride) : nullptr,
                                   hist ? (uint32_t)conv_dim * 12u : 0u);
        const auto tb = raw_buffer(const_cast<float *>(P.conv_w), conv ? (uint32_t)conv_dim * 16u : 0u);
        hq = __builtin_amdgcn_raw_buffer_load_b96(hb, (uint32_t)ch * 12u, 0, 0);
        wq = buf_load_f4(tb, (uint32_t)ch * 16u);
        hv = __builtin_amdgcn_raw_buffer_load_b96(hb, (uint32_t)chv * 12u, 0, 0);
        wv = buf_load_f4(tb, (uint32_t)chv * 16u);
        const E *zrow = norm ? static_cast<const E *>(P.z) + ((int64_t)i * P.H_v + h) * DV : nullptr;
        const auto zb = raw_buffer(const_cast<E *>(zrow), norm ? DV * sizeof(E) : 0u);
        if constexpr (sizeof(E) == 2)
            zs = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(zb, ev * 2u, 0, 0) << 16);
        else
            zs = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(zb, ev * 4u, 0, 0));
        nws = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            raw_buffer(const_cast<float *>(P.norm_w), norm ? DV * 4u : 0u), ev * 4u, 0, 0));
    }
    // the state block, last (zeros without a state)
    __builtin_amdgcn_sched_barrier(0);
    float4 s[RPT];
    {
        const auto sb = raw_buffer(sin >= 0 ? const_cast<float *>(P.state_in + (int64_t)sin * P.slot_stride +
                                                                  (int64_t)h * DK * DV)
                                            : nullptr,
                                   sin >= 0 ? (uint32_t)(DK * DV * 4) : 0u);
#pragma unroll
        for (int r = 0; r < RPT; ++r)   // one lane offset, the row step as the scalar offset
            s[r] = buf_load_f4(sb, (uint32_t)((rg * DV + col) * 4), (uint32_t)(r * RG * DV * 4));
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. gates and prologue, while the state streams in
    gi = P.gates.raw ? gate_g(gi, bias, rate) : gi;
    bi = P.gates.raw ? gate_beta(bi) : bi;
    float4 nqk = make_float4(0.f, 0.f, 0.f, 0.f), nvv = nqk;
    if (conv) {
        const float h0 = __uint_as_float(hq.x), h1 = __uint_as_float(hq.y), h2 = __uint_as_float(hq.z);
        nqk = make_float4(h1, h2, x, 0.f);
        x = conv1(wq, h0, h1, h2, x);
        const float g0 = __uint_as_float(hv.x), g1 = __uint_as_float(hv.y), g2 = __uint_as_float(hv.z);
        nvv = make_float4(g1, g2, xv, 0.f);
        xv = conv1(wv, g0, g1, g2, xv);
    }
    if (tid < 2 * DK) (isk ? sk : sq)[e] = x;
    if constexpr (FUSED) {
        if (tid < DV) {
            sv_[grp][ev] = xv;
            sz_[grp][ev] = norm ? nws * silu(zs) : 0.f;
        }
        // this thread's reads of the old convolution state are complete
        // before the barrier (x and xv are formed from them): after it, each
        // group's v channels and the key head's q and k channels take their
        // new state (no other workgroup reads them); lanes that do not write
        // get an offset past the range
        loaded(x);
        loaded(xv);
        lds_sync();
        const bool wr = conv && P.conv_out && sout >= 0;
        const auto cb = raw_buffer(wr ? P.conv_out + (int64_t)sout * P.slot_stride : nullptr,
                                   wr ? (uint32_t)conv_dim * 12u : 0u);
        const uint32_t vo = tid < DV ? (uint32_t)chv * 12u : kDropOffset;
        __builtin_amdgcn_raw_buffer_store_b96(
            u32x3{__float_as_uint(nvv.x), __float_as_uint(nvv.y), __float_as_uint(nvv.z)}, cb, vo, 0, 0);
        const uint32_t qo = grp == 0 && tid < 2 * DK ? (uint32_t)ch * 12u : kDropOffset;
        __builtin_amdgcn_raw_buffer_store_b96(
            u32x3{__float_as_uint(nqk.x), __float_as_uint(nqk.y), __float_as_uint(nqk.z)}, cb, qo, 0, 0);
        const float4 v4 = *reinterpret_cast<const float4 *>(&sv_[grp][col]);
        vv[0] = v4.x; vv[1] = v4.y; vv[2] = v4.z; vv[3] = v4.w;
    } else {
        lds_sync();
    }

    // 3. norms (every wave reduces redundantly; no extra barrier)
    float kk = 0.f, qq = 0.f, kq = 0.f;
    const int lane = tid & 63;
    for (int j = lane; j < DK; j += 64) {
        const float a = sk[j], b = sq[j];
        kk += a * a;
        qq += b * b;
        kq += a * b;
    }
    kk = group_sum<64>(kk);
    qq = group_sum<64>(qq);
    kq = group_sum<64>(kq);
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
    if (norm) {
        const float4 z4 = *reinterpret_cast<const float4 *>(&sz_[grp][col]);
        const float zg[4] = {z4.x, z4.y, z4.z, z4.w};
        gated_norm_row<CG, DV>(o, zg, P.eps);
    }

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

// Sum over the row groups of one wave: lanes that hold the same column group
// (lane mod CG) and different row groups, i.e. lanes l ^ 8 (CG = 8: a rotation
// by 8 within the row), l ^ 16 and l ^ 32 (the row swaps).
template <int CG>
__device__ __forceinline__ float rg_wave_sum(float x)
{
    if constexpr (CG <= 8) x = dpp_add<0x128>(x);      // row_ror:8
    if constexpr (CG <= 16) x = row_swap_add<1>(x);
    return row_swap_add<2>(x);
}

// Several tokens per sequence (speculative-decoding verification, short
// prompts): the same step, token after token, with the state block held in
// registers, so it is read from and written to HBM once per call instead of
// once per token.  q, k, v, g, beta (and z) of the next token are fetched
// while the current one is processed; k, q and the reduction partials
// alternate between two LDS buffers, so a token needs two barriers.  With the
// prologue, each thread keeps the convolution window of its q or k channel
// and of its v channel from token to token (in LDS slots of its own: registers
// are what limit this kernel).  FUSED (here and in decode_kernel):
// prologue and/or epilogue present; the plain instantiation carries none of
// their code or registers.
template <int DK, int DV, typename E, typename OT, bool FUSED, int GR>
__global__ __launch_bounds__(kDecodeThreads * GR, 4) void decode_multi_kernel(RecParams P)
{
    constexpr int CG = DV / 4;                  // float4 column groups
    constexpr int RG = kDecodeThreads / CG;     // row groups
    constexpr int RPT = DK / RG;                // state rows per thread
    static_assert(RPT >= 1 && RPT * RG == DK && 2 * DK <= kDecodeThreads, "bad decode tiling");

    const int i = blockIdx.x;                   // sequence
    const int grp = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kDecodeThreads);
    const int tid = (int)threadIdx.x % kDecodeThreads;
    const int cg = tid % CG;
    const int rg = tid / CG;
    const int col = cg * 4;
    const int h = GR > 1 ? (int)blockIdx.y * GR + grp : (int)blockIdx.y;   // value head
    const int kh = h / (P.H_v / P.H_k);
    const int lane = tid & 63;
    const E *q = static_cast<const E *>(P.q);
    const E *k = static_cast<const E *>(P.k);
    const E *v = static_cast<const E *>(P.v);
    const bool conv = FUSED && P.conv_w != nullptr;
    const bool norm = FUSED && P.z != nullptr;

    __shared__ float sk_[GR][2][DK];
    __shared__ float sq_[GR][2][DK];
    constexpr int NW = kDecodeThreads / 64;
    __shared__ float4 red_[GR][2][2][NW][CG];
    // fused: v after the prologue and w * silu(z) of a token, per channel
    __shared__ __attribute__((aligned(16))) float sv_[FUSED ? GR : 1][2][FUSED ? DV : 1];
    __shared__ __attribute__((aligned(16))) float sz_[FUSED ? GR : 1][2][FUSED ? DV : 1];
    // fused: the taps of this group's q / k channels and v channels, and the
    // norm weight, read per token (registers are what limit this kernel)
    // (one slot per thread: each thread reads back only what it wrote)
    __shared__ __attribute__((aligned(16))) float4 stq_[FUSED ? GR : 1][FUSED ? kDecodeThreads : 1];
    __shared__ __attribute__((aligned(16))) float4 stv_[FUSED ? GR : 1][FUSED ? kDecodeThreads : 1];
    __shared__ float snw_[FUSED ? GR : 1][FUSED ? kDecodeThreads : 1];
    // the convolution windows (the last three inputs of the q or k channel
    // and of the v channel), one slot per thread
    __shared__ float shw_[FUSED ? GR : 1][FUSED ? 6 : 1][FUSED ? kDecodeThreads : 1];
    float(&sk)[2][DK] = sk_[grp];
    float(&sq)[2][DK] = sq_[grp];
    float4(&red)[2][2][NW][CG] = red_[grp];

    // tokens of this sequence (clamped so that bad cu_seqlens stay in range)
    const int tb = min(max(P.cu[i], 0), P.T);
    const int te = min(max(P.cu[i + 1], tb), P.T);
    const int sin = P.state_in ? P.slot_in[i] : -1;
    const int sout = P.slot_out[i];

    // this thread's channels: one q or k channel of the key head (threads
    // past 2 DK repeat one) and, fused, one v channel (threads past DV repeat
    // one); plain, four v columns
    const int e2 = tid % (2 * DK);
    const bool isk = e2 < DK;
    const int e = isk ? e2 : e2 - DK;
    const int ev = tid % DV;
    const int conv_dim = 2 * P.H_k * DK + P.H_v * DV;
    const int64_t chq = (isk ? (int64_t)P.H_k * DK : 0) + (int64_t)kh * DK + e;
    const int64_t chv = 2 * (int64_t)P.H_k * DK + (int64_t)h * DV + ev;

    // Order of memory operations as in decode_kernel: the prologue's taps and
    // stored inputs, the norm weight and the first token are loaded before
    // the state block, and a token's inputs are only fetched, so the next
    // token's loads stay in flight while the current one is processed.
    u32x3 hq3 = {0u, 0u, 0u}, hv3 = {0u, 0u, 0u};
    float4 wq = make_float4(0.f, 0.f, 0.f, 0.f), wv = wq;
    float nws = 0.f;
    if constexpr (FUSED) {
        const bool hist = conv && sin >= 0;
        const auto hb = raw_buffer(hist ? const_cast<float *>(P.conv_in + (int64_t)sin * P.slot_stride) : nullptr,
                                   hist ? (uint32_t)conv_dim * 12u : 0u);
        const auto tbuf = raw_buffer(const_cast<float *>(P.conv_w), conv ? (uint32_t)conv_dim * 16u : 0u);
        hq3 = __builtin_amdgcn_raw_buffer_load_b96(hb, (uint32_t)chq * 12u, 0, 0);
        wq = buf_load_f4(tbuf, (uint32_t)chq * 16u);
        hv3 = __builtin_amdgcn_raw_buffer_load_b96(hb, (uint32_t)chv * 12u, 0, 0);
        wv = buf_load_f4(tbuf, (uint32_t)chv * 16u);
        nws = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            raw_buffer(const_cast<float *>(P.norm_w), norm ? DV * 4u : 0u), ev * 4u, 0, 0));
    }

    // a token's inputs for this thread: its q or k value and v (fused: its
    // channel and z; plain: four columns)
    struct Tok {
        float kq;
        float vv[4];
        float zs;
    };
    auto fetch = [&](int t) {
        Tok r;
        r.kq = to_f32((isk ? k : q)[(int64_t)t * P.rs_qk + (int64_t)kh * DK + e]);
        const E *vrow = v + (int64_t)t * P.rs_v + (int64_t)h * DV;
        if constexpr (FUSED) {
            r.vv[0] = to_f32(vrow[ev]);
            r.vv[1] = r.vv[2] = r.vv[3] = 0.f;
            const E *zrow = norm ? static_cast<const E *>(P.z) + ((int64_t)t * P.H_v + h) * DV : nullptr;
            const auto zb = raw_buffer(const_cast<E *>(zrow), norm ? DV * sizeof(E) : 0u);
            if constexpr (sizeof(E) == 2)
                r.zs = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(zb, ev * 2u, 0, 0) << 16);
            else
                r.zs = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(zb, ev * 4u, 0, 0));
        } else {
            buf_load4<E>(raw_buffer(const_cast<E *>(vrow), DV * sizeof(E)), col * sizeof(E), r.vv);
            r.zs = 0.f;
        }
        return r;
    };
    // g and beta of up to 64 tokens per wave: lane l holds those of token
    // tb + base + l (the last token's past the end).  A batch is activated
    // once, all its tokens at once, and each token takes its pair with a
    // lane read: activated per token in every thread, the raw gates (two
    // exponentials, a logarithm and a division) cost more vector-ALU time
    // than the token's state arithmetic leaves free.
    float gl = 0.f, bl = 0.f;
    auto gate_load = [&](int base) {
        const int64_t t = min(tb + base + lane, te - 1);
        gl = P.g[t * P.H_v + h];
        bl = P.beta[t * P.H_v + h];
    };
    Tok cur{};
    float rate = 0.f, bias = 0.f;
    if (tb < te) {                              // an empty sequence reads no token
        cur = fetch(tb);
        gate_load(0);
        rate = P.gates.rate[h];
        bias = P.gates.bias[h];
    }

    // the state block, last.  Fused: through a buffer resource (zeros
    // without a state, no branch).  Plain: global loads behind a branch; the
    // buffer form would cost this instantiation about 20 registers and a
    // wave per SIMD, more than the branch costs it.
    __builtin_amdgcn_sched_barrier(0);
    float4 s[RPT];
    if constexpr (FUSED) {
        const auto sb = raw_buffer(sin >= 0 ? const_cast<float *>(P.state_in + (int64_t)sin * P.slot_stride +
                                                                  (int64_t)h * DK * DV)
                                            : nullptr,
                                   sin >= 0 ? (uint32_t)(DK * DV * 4) : 0u);
#pragma unroll
        for (int r = 0; r < RPT; ++r)   // one lane offset, the row step as the scalar offset
            s[r] = buf_load_f4(sb, (uint32_t)((rg * DV + col) * 4), (uint32_t)(r * RG * DV * 4));
    } else if (sin >= 0) {
        const float *base = P.state_in + (int64_t)sin * P.slot_stride + (int64_t)h * DK * DV + col;
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            s[r] = *reinterpret_cast<const float4 *>(base + (int64_t)(rg + r * RG) * DV);
    } else {
#pragma unroll
        for (int r = 0; r < RPT; ++r) s[r] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __builtin_amdgcn_sched_barrier(0);

    if constexpr (FUSED) {
        stq_[grp][tid] = wq;
        stv_[grp][tid] = wv;
        snw_[grp][tid] = nws;
    }
    // convolution windows: the last three inputs of each channel
    if constexpr (FUSED) {
        shw_[grp][0][tid] = __uint_as_float(hq3.x);
        shw_[grp][1][tid] = __uint_as_float(hq3.y);
        shw_[grp][2][tid] = __uint_as_float(hq3.z);
        shw_[grp][3][tid] = __uint_as_float(hv3.x);
        shw_[grp][4][tid] = __uint_as_float(hv3.y);
        shw_[grp][5][tid] = __uint_as_float(hv3.z);
    }
    // fused: the per-head gate parameters in scalar registers (their loads
    // were issued before the state block's branch-free loads, so this waits
    // for nothing later; after the plain kernel's branch it would wait for
    // the whole block)
    // (the builtin takes an int: the bits pass through it, not the value)
    if constexpr (FUSED) {
        rate = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(rate)));
        bias = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(bias)));
    }

    for (int t = tb; t < te; ++t) {
        const int b = (t - tb) & 1;
        const int j = (t - tb) & 63;
        if (j == 0) {
            if (t != tb) gate_load(t - tb);
            if (P.gates.raw) {
                gl = gate_g(gl, bias, rate);
                bl = gate_beta(bl);
            }
        }
        const float gt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gl), j));
        const float bt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bl), j));
        float kqv = cur.kq;
        if (conv) {
            const float h0 = shw_[grp][0][tid], h1 = shw_[grp][1][tid], h2 = shw_[grp][2][tid];
            kqv = conv1(stq_[grp][tid], h0, h1, h2, cur.kq);
            shw_[grp][0][tid] = h1; shw_[grp][1][tid] = h2; shw_[grp][2][tid] = cur.kq;
        }
        if (tid < 2 * DK) (isk ? sk[b] : sq[b])[e] = kqv;
        if constexpr (FUSED) {
            float xv = cur.vv[0];
            if (conv) {
                const float h0 = shw_[grp][3][tid], h1 = shw_[grp][4][tid], h2 = shw_[grp][5][tid];
                xv = conv1(stv_[grp][tid], h0, h1, h2, cur.vv[0]);
                shw_[grp][3][tid] = h1; shw_[grp][4][tid] = h2; shw_[grp][5][tid] = cur.vv[0];
            }
            if (tid < DV) {
                sv_[grp][b][ev] = xv;
                sz_[grp][b][ev] = norm ? snw_[grp][tid] * silu(cur.zs) : 0.f;
            }
        }
        const Tok nxt = fetch(min(t + 1, te - 1));
        lds_sync();
        float vv[4] = {cur.vv[0], cur.vv[1], cur.vv[2], cur.vv[3]};
        if constexpr (FUSED) {
            const float4 v4 = *reinterpret_cast<const float4 *>(&sv_[grp][b][col]);
            vv[0] = v4.x; vv[1] = v4.y; vv[2] = v4.z; vv[3] = v4.w;
        }

        // norms (every wave reduces redundantly; no extra barrier)
        float kk = 0.f, qq = 0.f, kq = 0.f;
        for (int j = lane; j < DK; j += 64) {
            const float a = sk[b][j], c = sq[b][j];
            kk += a * a;
            qq += c * c;
            kq += a * c;
        }
        kk = group_sum<64>(kk);
        qq = group_sum<64>(qq);
        kq = group_sum<64>(kq);
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
        const float dec = expf(gt);
        const float dk_ = dec * rk;
        float4 d;
        d.x = bt * (vv[0] - dk_ * tk.x);
        d.y = bt * (vv[1] - dk_ * tk.y);
        d.z = bt * (vv[2] - dk_ * tk.z);
        d.w = bt * (vv[3] - dk_ * tk.w);
        const float dq = dec * rq, kqh = rk * rq * kq;
        float o[4] = {dq * tq.x + kqh * d.x, dq * tq.y + kqh * d.y, dq * tq.z + kqh * d.z,
                      dq * tq.w + kqh * d.w};
        if (norm) {
            const float4 z4 = *reinterpret_cast<const float4 *>(&sz_[grp][b][col]);
            const float zg[4] = {z4.x, z4.y, z4.z, z4.w};
            gated_norm_row<CG, DV>(o, zg, P.eps);
        }
        {
            // row group 0 writes the row; the other lanes' offsets fall past
            // the buffer's end and are dropped.  No branch: a store inside one
            // would make the next wait for the prefetched token wait for it
            // too (on gfx9 stores and loads share the counter).
            const __amdgpu_buffer_rsrc_t ob =
                raw_buffer(static_cast<OT *>(P.out) + ((int64_t)t * P.H_v + h) * DV, (uint32_t)(DV * sizeof(OT)));
            const uint32_t off = rg == 0 ? (uint32_t)(col * sizeof(OT)) : kDropOffset;
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

    if constexpr (FUSED) {
        if (conv && P.conv_out) {
            // The windows hold the last three inputs of each channel (the old
            // state shifted by the sequence's rows): the new convolution
            // state.  This thread's reads of the old state are complete
            // before the barrier (the windows are formed from them); each
            // group's v channels and the key head's q and k channels are read
            // by no other workgroup.
            float hq[3], hv[3];
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                hq[j] = shw_[grp][j][tid];
                hv[j] = shw_[grp][3 + j][tid];
                loaded(hq[j]);
                loaded(hv[j]);
            }
            lds_sync();
            const auto cb = raw_buffer(sout >= 0 ? P.conv_out + (int64_t)sout * P.slot_stride : nullptr,
                                       sout >= 0 ? (uint32_t)conv_dim * 12u : 0u);
            const uint32_t vo = tid < DV ? (uint32_t)chv * 12u : kDropOffset;
            __builtin_amdgcn_raw_buffer_store_b96(
                u32x3{__float_as_uint(hv[0]), __float_as_uint(hv[1]), __float_as_uint(hv[2])}, cb, vo, 0, 0);
            const uint32_t qo = grp == 0 && tid < 2 * DK ? (uint32_t)chq * 12u : kDropOffset;
            __builtin_amdgcn_raw_buffer_store_b96(
                u32x3{__float_as_uint(hq[0]), __float_as_uint(hq[1]), __float_as_uint(hq[2])}, cb, qo, 0, 0);
        }
    }
    if (sout >= 0) {
        float *base = P.state_out + (int64_t)sout * P.slot_stride + (int64_t)h * DK * DV + col;
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            *reinterpret_cast<float4 *>(base + (int64_t)(rg + r * RG) * DV) = s[r];
    }
}

// Value heads per workgroup with the prologue: H_v / H_k when it is 1 or 2,
// else 0 (one value head per workgroup, the state left to
// conv_state_kernel).  Four groups would not fit the kernels' registers into
// the 128 per thread of a 1024-thread workgroup.
int conv_groups(const Problem &p)
{
    const int r = p.H_v / p.H_k;
    return r == 1 || r == 2 ? r : 0;
}

template <int DK, int DV, typename E, typename OT>
hipError_t launch_multi_t(const Problem &p, const DecodeMultiArgs &a, hipStream_t st)
{
    const RecParams P = rec_params(p, a.q, a.k, a.v, a.g, a.beta, a.state_in, a.state_out, a.out,
                                   a.cu_seqlens, a.slot_in, a.slot_out, (int)a.total_tokens, a.conv_in,
                                   decode_folds_conv(p) ? a.conv_out : nullptr);
    if (!p.conv_w && !p.z)
        hipLaunchKernelGGL((decode_multi_kernel<DK, DV, E, OT, false, 1>), dim3(a.n_seqs, p.H_v),
                           dim3(kDecodeThreads), 0, st, P);
    else if (p.conv_w && conv_groups(p) == 2)
        hipLaunchKernelGGL((decode_multi_kernel<DK, DV, E, OT, true, 2>), dim3(a.n_seqs, p.H_k),
                           dim3(2 * kDecodeThreads), 0, st, P);
    else
        hipLaunchKernelGGL((decode_multi_kernel<DK, DV, E, OT, true, 1>), dim3(a.n_seqs, p.H_v),
                           dim3(kDecodeThreads), 0, st, P);
    return hipGetLastError();
}

template <int DK, int DV, typename E, typename OT>
hipError_t launch_t(const Problem &p, const DecodeArgs &a, hipStream_t st)
{
    const RecParams P = rec_params(p, a.q, a.k, a.v, a.g, a.beta, a.state_in, a.state_out, a.out,
                                   nullptr, a.slot_in, a.slot_out, a.n_seqs, a.conv_in,
                                   decode_folds_conv(p) ? a.conv_out : nullptr);
    if (!p.conv_w && !p.z)
        hipLaunchKernelGGL((decode_kernel<DK, DV, E, OT, false, 1>), dim3(a.n_seqs, p.H_v), dim3(kDecodeThreads),
                           0, st, P);
    else if (p.conv_w && conv_groups(p) == 2)
        hipLaunchKernelGGL((decode_kernel<DK, DV, E, OT, true, 2>), dim3(a.n_seqs, p.H_k),
                           dim3(2 * kDecodeThreads), 0, st, P);
    else
        hipLaunchKernelGGL((decode_kernel<DK, DV, E, OT, true, 1>), dim3(a.n_seqs, p.H_v), dim3(kDecodeThreads),
                           0, st, P);
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

bool decode_folds_conv(const Problem &p)
{
    return p.conv_w && conv_groups(p) != 0;
}

hipError_t launch_decode(const Problem &p, const DecodeArgs &a, hipStream_t st)
{
    return launch_any<DecodeArgs, false>(p, a, st);
}

hipError_t launch_decode_multi(const Problem &p, const DecodeMultiArgs &a, hipStream_t st)
{
    return launch_any<DecodeMultiArgs, true>(p, a, st);
}

}  // namespace gdn
