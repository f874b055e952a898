// gdn_prefill.hip -- chunked (64-token) prefill of the gated delta rule on
// gfx950 matrix cores.
//
// The chunked WY form is the one the page "Optimization: Qwen3 next
// autoregressive pass (#17996)" builds in build_delta_net_chunking (and, for
// one chunk, in the body of the removed build_delta_net_recurrent).  For a
// chunk of n <= 64 tokens with incoming state S (d_k x d_v):
//
//   G_r   = inclusive cumsum of g                          (g_cumsum)
//   Gam   = exp(G_r - G_c) for c <= r, else 0              (decay_mask)
//   A     = strict_lower(diag(beta) (K^ K^T) * Gam)        (-attn before solve)
//   T     = (I + A)^-1                                     (solve_tri + identity)
//   W     = T diag(beta e^G) K^                            (k_cumdecay)
//   U     = T diag(beta) V - W S                           (value - v_prime = v_new)
//   O     = diag(e^G) Q^ S + (Q^ K^T * Gam) U              (attn_inter + v_attn)
//   S_out = e^{G_n} S + K^T diag(e^{G_n - G}) U            (new state)
//
// MI355X mapping (three launches):
//   1. chunk_table_kernel: cu_seqlens -> one descriptor per 64-token chunk
//      (sequence, first token, length) and each sequence's chunk range.
//   2. prep_kernel, one workgroup per (chunk, key head): everything that does
//      not depend on the carried state, for all value heads sharing the key
//      head: K K^T and K Q^T once (bf16 MFMA, fp32 accumulate), the decay
//      masks from an fp64 cumulative sum (so exp(G_r - G_c) never forms a
//      factor exp(-G) that would overflow), T by blocked forward substitution
//      in LDS (16x16 diagonal blocks by substitution, off-diagonal blocks with
//      fp32 MFMA), then W.  T diag(beta), W and the masked attention are
//      written to the workspace as ready-made MFMA operand fragments.
//   3. scan_kernel, one workgroup per (sequence, value head, 16*NW value
//      columns): walks the sequence's chunks in order with the state held in
//      MFMA accumulator registers for the whole sequence (never round-tripped
//      through HBM between chunks).  Per chunk: U = T'V - W S, the output
//      O = qs*(Q S) + P U, and S = gn*S + K^T (ks*U).  Each wave owns 16 state
//      columns, so every product on the state chain is wave-local.
//
// Norms, scale, beta and decay are folded into per-row / per-column scalars
// of raw (bf16) operands, so the inputs are used as MFMA operands exactly as
// stored.  A final partial chunk is zero-padded; padded rows carry beta = 0,
// g = 0 and zero norms, which makes them the identity on the state.
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

constexpr int C = kChunk;

struct ChunkEntry {
    int32_t seq, t0, len, pad;
};

__host__ __device__ constexpr int kb_of(bool bf16) { return bf16 ? 32 : 16; }

// Per (chunk, value head) workspace block, in 1 KiB fragments:
//   W (4 x d_k/KB) | T' hi [| T' lo] | P hi [| P lo] | scalars (qs, ks, gn)
// (the lo halves exist for bf16 operands only).
__host__ __device__ constexpr int n_split(bool bf16) { return bf16 ? 2 : 1; }
__host__ __device__ constexpr int n_wfrag(int d_k, bool bf16) { return 4 * (d_k / kb_of(bf16)); }
__host__ __device__ constexpr int n_tfrag(bool bf16) { return 4 * (C / kb_of(bf16)); }
__host__ __device__ constexpr size_t block_bytes(int d_k, bool bf16) {
    return (size_t)(n_wfrag(d_k, bf16) + 2 * n_split(bf16) * n_tfrag(bf16)) * 1024 + 1024;
}

struct WsLayout {
    size_t entries, cstart, blocks, block, total;
    int max_chunks;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

WsLayout ws_layout(const Problem &p, int32_t n_seqs, int64_t T)
{
    WsLayout L;
    L.max_chunks = (int)max_chunks(n_seqs, T);
    L.entries = 256;
    L.cstart = align256(L.entries + sizeof(ChunkEntry) * (size_t)L.max_chunks);
    L.blocks = align256(L.cstart + sizeof(int32_t) * ((size_t)n_seqs + 1));
    L.block = block_bytes(p.d_k, p.bf16 != 0);
    L.total = L.blocks + L.block * (size_t)L.max_chunks * p.H_v;
    return L;
}

// --------------------------------------------------------------------------
// 1. chunk table
// --------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void chunk_table_kernel(
    const int32_t *__restrict__ cu, int n_seqs, int T, int max_ch,
    int32_t *__restrict__ hdr, ChunkEntry *__restrict__ ent, int32_t *__restrict__ cstart)
{
    __shared__ int wsum[16];
    __shared__ int s_carry;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    if (tid == 0) s_carry = 0;
    __syncthreads();
    for (int base = 0; base < n_seqs; base += 1024) {
        const int i = base + tid;
        int tb = 0, te = 0;
        if (i < n_seqs) {        // clamp so that bad cu_seqlens never index out of range
            tb = min(max(cu[i], 0), T);
            te = min(max(cu[i + 1], tb), T);
        }
        const int nc = (te - tb + C - 1) / C;
        int x = nc;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        if (lane == 63) wsum[wid] = x;
        __syncthreads();
        int before = 0, total = 0;
        for (int w = 0; w < 16; ++w) {
            total += wsum[w];
            if (w < wid) before += wsum[w];
        }
        const int carry = s_carry;
        const int start = carry + before + x - nc;
        if (i < n_seqs) {
            cstart[i] = min(start, max_ch);
            for (int c = 0; c < nc; ++c) {
                const int idx = start + c;
                if (idx < max_ch) {
                    ChunkEntry e;
                    e.seq = i;
                    e.t0 = tb + c * C;
                    e.len = min(C, te - tb - c * C);
                    e.pad = 0;
                    ent[idx] = e;
                }
            }
        }
        __syncthreads();
        if (tid == 0) s_carry = carry + total;
        __syncthreads();
    }
    if (tid == 0) {
        const int n = min(s_carry, max_ch);
        cstart[n_seqs] = n;
        hdr[0] = n;
    }
}

// --------------------------------------------------------------------------
// helpers
// --------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return (uint32_t)bf16_bits_rne(a) | ((uint32_t)bf16_bits_rne(b) << 16);
}

// Write 4 consecutive k-values (one accumulator column) into half `half` of
// fragment f: 8 bytes (bf16) or 16 bytes (fp32) at the lane's slot.
template <typename E> __device__ __forceinline__ void store_quarter(void *base, int f, int lane, int half, floatx4 v);
template <> __device__ __forceinline__ void store_quarter<bf16_t>(void *base, int f, int lane, int half, floatx4 v) {
    uint2 u = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    *reinterpret_cast<uint2 *>(reinterpret_cast<char *>(base) + ((size_t)f * 64 + lane) * 16 + half * 8) = u;
}
template <> __device__ __forceinline__ void store_quarter<float>(void *base, int f, int lane, int half, floatx4 v) {
    (void)half;
    *reinterpret_cast<floatx4 *>(reinterpret_cast<char *>(base) + ((size_t)f * 64 + lane) * 16) = v;
}

// Same, for a two-term operand: hi into `hi_base`, lo into `lo_base`.
template <typename E> __device__ __forceinline__ void store_quarter2(void *hi_base, void *lo_base, int f, int lane, int half, floatx4 v);
template <> __device__ __forceinline__ void store_quarter2<bf16_t>(void *hi_base, void *lo_base, int f, int lane, int half, floatx4 v) {
    floatx4 h, l;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        h[j] = __uint_as_float((uint32_t)bf16_bits_rne(v[j]) << 16);
        l[j] = v[j] - h[j];
    }
    store_quarter<bf16_t>(hi_base, f, lane, half, h);
    store_quarter<bf16_t>(lo_base, f, lane, half, l);
}
template <> __device__ __forceinline__ void store_quarter2<float>(void *hi_base, void *lo_base, int f, int lane, int half, floatx4 v) {
    (void)lo_base;
    store_quarter<float>(hi_base, f, lane, half, v);
}

template <typename E> struct ElemVec;
template <> struct ElemVec<bf16_t> {
    static constexpr int N = 8;
    __device__ static __forceinline__ float get(const uint4 &u, int e) {
        const uint32_t w = (&u.x)[e >> 1];
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    __device__ static __forceinline__ bf16_t raw(const uint4 &u, int e) {
        const uint32_t w = (&u.x)[e >> 1];
        bf16_t r;
        r.bits = (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu));
        return r;
    }
};
template <> struct ElemVec<float> {
    static constexpr int N = 4;
    __device__ static __forceinline__ float get(const uint4 &u, int e) { return __uint_as_float((&u.x)[e]); }
    __device__ static __forceinline__ float raw(const uint4 &u, int e) { return __uint_as_float((&u.x)[e]); }
};

// lower 16x16 tile pairs (rt, ct), ct <= rt, and the strictly upper ones
__constant__ int kLowR[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ int kLowC[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
__constant__ int kUpR[6] = {0, 0, 0, 1, 1, 2};
__constant__ int kUpC[6] = {1, 2, 3, 2, 3, 3};

struct PrepParams {
    const void *q, *k;
    const float *g, *beta;
    const int32_t *hdr;
    const ChunkEntry *ent;
    char *blocks;
    size_t block;
    int H_k, H_v;
    float scale, eps;
};

template <int DK, typename E> struct PrepLds {
    static constexpr int VEC = 16 / (int)sizeof(E);
    static constexpr int LDK = DK + VEC;     // row-major K, Q (elements)
    static constexpr int LDT = C + VEC;      // transposed K
    static constexpr int LDA = C + 4;        // fp32 A and T
    static constexpr size_t R1a = 2ull * C * LDK * sizeof(E);
    static constexpr size_t R1b = 2ull * C * LDA * sizeof(float);
    static constexpr size_t R1 = R1a > R1b ? R1a : R1b;
    static constexpr size_t R2 = (size_t)DK * LDT * sizeof(E);
    static constexpr size_t R2p = (R2 + 15) / 16 * 16;
    static constexpr size_t SMALL = C * sizeof(double) + 5 * C * sizeof(float);
    static constexpr size_t BYTES = R1 + R2p + SMALL;
};

// --------------------------------------------------------------------------
// 2. per-chunk preparation (state independent)
// --------------------------------------------------------------------------
template <int DK, typename E>
__global__ __launch_bounds__(256) void prep_kernel(PrepParams pp)
{
    using M = Mfma<E>;
    using SP = Split<E>;
    using L = PrepLds<DK, E>;
    using V = ElemVec<E>;
    constexpr int KB = M::KB, TPB = M::TPB, VEC = L::VEC, NS = SP::N;
    constexpr int LDK = L::LDK, LDT = L::LDT, LDA = L::LDA;
    constexpr int NKD = DK / KB, NKC = C / KB;
    constexpr int NWF = 4 * NKD, NTF = 4 * NKC;
    constexpr int VPR = DK / VEC;

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    E *sK = reinterpret_cast<E *>(smem);
    E *sQ = sK + C * LDK;
    float *sA = reinterpret_cast<float *>(smem);
    float *sT = sA + C * LDA;
    E *sKT = reinterpret_cast<E *>(smem + L::R1);
    double *sG = reinterpret_cast<double *>(smem + L::R1 + L::R2p);
    float *sBeta = reinterpret_cast<float *>(sG + C);
    float *srk = sBeta + C;
    float *srq = srk + C;
    float *scol = srq + C;

    const int chunk = blockIdx.x, kh = blockIdx.y;
    if (chunk >= pp.hdr[0]) return;
    const ChunkEntry ce = pp.ent[chunk];
    const int t0 = ce.t0, len = ce.len;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n = lane & 15, qd = lane >> 4;
    const E *qg = static_cast<const E *>(pp.q);
    const E *kg = static_cast<const E *>(pp.k);

    // 1. stage K, Q (row-major) and K^T; inverse row norms
    for (int vi = tid; vi < C * VPR; vi += 256) {
        const int r = vi / VPR, cv = vi % VPR;
        uint4 kv = make_uint4(0, 0, 0, 0), qv = kv;
        if (r < len) {
            const size_t off = ((size_t)(t0 + r) * pp.H_k + kh) * DK + (size_t)cv * VEC;
            kv = *reinterpret_cast<const uint4 *>(kg + off);
            qv = *reinterpret_cast<const uint4 *>(qg + off);
        }
        *reinterpret_cast<uint4 *>(sK + r * LDK + cv * VEC) = kv;
        *reinterpret_cast<uint4 *>(sQ + r * LDK + cv * VEC) = qv;
        float k2 = 0.f, q2 = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            sKT[(cv * VEC + e) * LDT + r] = V::raw(kv, e);
            const float a = V::get(kv, e), b = V::get(qv, e);
            k2 += a * a;
            q2 += b * b;
        }
#pragma unroll
        for (int off = VPR / 2; off >= 1; off >>= 1) {
            k2 += __shfl_xor(k2, off, 64);
            q2 += __shfl_xor(q2, off, 64);
        }
        if (cv == 0) {
            srk[r] = r < len ? rsqrtf(k2 + pp.eps) : 0.f;
            srq[r] = r < len ? rsqrtf(q2 + pp.eps) * pp.scale : 0.f;
        }
    }
    __syncthreads();

    // 2. raw K K^T (lower tiles) and K Q^T (tiles (ct, rt), ct <= rt): 20
    //    tile products, 5 per wave; kept in registers for all value heads.
    floatx4 acc[5];
#pragma unroll
    for (int s = 0; s < 5; ++s) {
        acc[s] = floatx4{0.f, 0.f, 0.f, 0.f};
        const int it = w + 4 * s;
        const int pr = it < 10 ? it : it - 10;
        const int rt = kLowR[pr], ct = kLowC[pr];
        const E *ra = it < 10 ? sK + (16 * rt + n) * LDK : sK + (16 * ct + n) * LDK;
        const E *rb = it < 10 ? sK + (16 * ct + n) * LDK : sQ + (16 * rt + n) * LDK;
#pragma unroll
        for (int kb = 0; kb < NKD; ++kb)
            M::mma(acc[s], M::load_rm(ra, kb * KB, qd), M::load_rm(rb, kb * KB, qd));
    }
    __syncthreads();   // sK / sQ are dead from here on (sA / sT alias them)

    const int ratio = pp.H_v / pp.H_k;
    for (int jv = 0; jv < ratio; ++jv) {
        const int h = kh * ratio + jv;
        char *blk = pp.blocks + ((size_t)chunk * pp.H_v + h) * pp.block;
        char *Wf = blk;
        char *Tf = blk + NWF * 1024;                    // T' hi, then T' lo
        char *Pf = blk + (NWF + NS * NTF) * 1024;       // P hi, then P lo
        float *scal = reinterpret_cast<float *>(blk + (NWF + 2 * NS * NTF) * 1024);

        // 3a. cumulative log-decay in fp64, per-row scalars
        if (w == 0) {
            const int r = lane;
            float gv = 0.f, bv = 0.f;
            if (r < len) {
                gv = pp.g[(size_t)(t0 + r) * pp.H_v + h];
                bv = pp.beta[(size_t)(t0 + r) * pp.H_v + h];
            }
            double G = gv;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const double y = __shfl_up(G, off, 64);
                if (lane >= off) G += y;
            }
            const double Gn = __shfl(G, 63, 64);
            sG[r] = G;
            sBeta[r] = bv;
            const float eG = expf((float)G);
            scal[r] = srq[r] * eG;                              // qs: q scale * e^{G_r}
            scal[64 + r] = srk[r] * expf((float)(Gn - G));      // ks: e^{G_n - G_r} / |k_r|
            if (r == 0) scal[128] = expf((float)Gn);            // gn: e^{G_n}
            scol[r] = bv * eG * srk[r];                         // columns of T'' = T diag(beta e^G / |k|)
        }
        __syncthreads();

        // 3b. A (strictly lower) -> LDS; masked, decayed Q.K -> P fragments
#pragma unroll
        for (int s = 0; s < 5; ++s) {
            const int it = w + 4 * s;
            if (it < 10) {
                const int rt = kLowR[it], ct = kLowC[it];
                const int c = 16 * ct + n;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * rt + 4 * qd + j;
                    float val = 0.f;
                    if (c < r)
                        val = sBeta[r] * srk[r] * srk[c] * acc[s][j] * expf((float)(sG[r] - sG[c]));
                    sA[r * LDA + c] = val;
                }
            } else {
                const int pr = it - 10;
                const int rt = kLowR[pr], ct = kLowC[pr];
                const int r = 16 * rt + n;
                floatx4 pv;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = 16 * ct + 4 * qd + j;
                    pv[j] = (c <= r) ? srq[r] * srk[c] * acc[s][j] * expf((float)(sG[r] - sG[c])) : 0.f;
                }
                store_quarter2<E>(Pf, Pf + NTF * 1024, rt * NKC + ct / TPB, lane, ct % TPB, pv);
            }
        }
        for (int z = w; z < 6; z += 4) {
            const int rt = kUpR[z], ct = kUpC[z];
            store_quarter2<E>(Pf, Pf + NTF * 1024, rt * NKC + ct / TPB, lane, ct % TPB,
                              floatx4{0.f, 0.f, 0.f, 0.f});
        }
        __syncthreads();

        // 3c. T = (I + A)^-1: diagonal 16x16 blocks by forward substitution
        //     (wave 0, one lane per column); other waves zero the upper blocks.
        if (w == 0) {
            const int b = lane >> 4, j = lane & 15;
            const float *Ab = sA + (16 * b) * LDA + 16 * b;
            float t[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float a = (i == j) ? 1.f : 0.f;
#pragma unroll
                for (int c = 0; c < i; ++c) a -= Ab[i * LDA + c] * t[c];
                t[i] = a;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sT[(16 * b + i) * LDA + 16 * b + j] = t[i];
        } else {
            for (int e = tid - 64; e < 6 * 256; e += 192) {
                const int z = e >> 8, within = e & 255;
                sT[(16 * kUpR[z] + (within >> 4)) * LDA + 16 * kUpC[z] + (within & 15)] = 0.f;
            }
        }
        __syncthreads();
        //     off-diagonal blocks by distance: T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj
        for (int d = 1; d < 4; ++d) {
            if (w < 4 - d) {
                const int bi = w + d, bj = w;
                floatx4 X = {0.f, 0.f, 0.f, 0.f};
                for (int m = bj; m < bi; ++m) {
                    const float4 av = *reinterpret_cast<const float4 *>(sA + (16 * bi + n) * LDA + 16 * m + 4 * qd);
                    floatx4 a = {av.x, av.y, av.z, av.w};
                    floatx4 bt;
#pragma unroll
                    for (int j = 0; j < 4; ++j) bt[j] = sT[(16 * m + 4 * qd + j) * LDA + 16 * bj + n];
                    mma_f32_k16(X, a, bt);
                }
                const float4 tv = *reinterpret_cast<const float4 *>(sT + (16 * bi + n) * LDA + 16 * bi + 4 * qd);
                floatx4 a = {-tv.x, -tv.y, -tv.z, -tv.w};
                floatx4 Y = {0.f, 0.f, 0.f, 0.f};
                mma_f32_k16(Y, a, X);
#pragma unroll
                for (int j = 0; j < 4; ++j) sT[(16 * bi + 4 * qd + j) * LDA + 16 * bj + n] = Y[j];
            }
            __syncthreads();
        }

        // 3d. T' = T diag(beta) as (two-term) A-operand fragments (rows r, k = c)
        for (int f = w; f < NTF; f += 4) {
            const int rt = f / NKC, kb = f % NKC;
            typename M::Frag hi, lo;
            SP::rm_f32(sT + (16 * rt + n) * LDA, kb * KB, qd, sBeta, hi, lo);
            store_frag<E>(Tf, f, lane, hi);
            if constexpr (NS == 2) store_frag<E>(Tf + NTF * 1024, f, lane, lo);
        }
        //     W^T = K^T T''^T tiles (dk tile dt, token tile tt) -> W fragments
        for (int item = w; item < (DK / 16) * 4; item += 4) {
            const int dt = item % (DK / 16), tt = item / (DK / 16);
            floatx4 a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb) {
                if (kb * KB > 16 * tt + 15) break;
                const typename M::Frag a = M::load_rm(sKT + (16 * dt + n) * LDT, kb * KB, qd);
                typename M::Frag hi, lo;
                SP::rm_f32(sT + (16 * tt + n) * LDA, kb * KB, qd, scol, hi, lo);
                M::mma(a4, a, hi);
                if constexpr (NS == 2) M::mma(a4, a, lo);
            }
            store_quarter<E>(Wf, tt * NKD + dt / TPB, lane, dt % TPB, a4);
        }
        __syncthreads();
    }
}

// --------------------------------------------------------------------------
// 3. sequential state scan + output
// --------------------------------------------------------------------------
struct ScanParams {
    const void *q, *k, *v;
    const float *state_in;
    float *state_out;
    void *out;
    const int32_t *slot_in, *slot_out;
    const int32_t *cstart;
    const ChunkEntry *ent;
    const char *blocks;
    size_t block;
    int H_k, H_v;
    int64_t slot_stride;
};

template <int DK, int NW, typename E> struct ScanLds {
    static constexpr int VEC = 16 / (int)sizeof(E);
    static constexpr int DVB = 16 * NW;
    static constexpr int LDQ = DK + VEC;
    static constexpr int LDT = C + VEC;
    static constexpr size_t Q = (size_t)C * LDQ * sizeof(E);
    static constexpr size_t KT = (size_t)DK * LDT * sizeof(E);
    static constexpr size_t VT = (size_t)DVB * LDT * sizeof(E);
    static constexpr size_t BYTES = Q + KT + VT + 3 * C * sizeof(float);
};

template <int DK, int DV, int NW, typename E, typename OT>
__global__ __launch_bounds__(NW * 64) void scan_kernel(ScanParams sp)
{
    using M = Mfma<E>;
    using SP = Split<E>;
    using Frag = typename M::Frag;
    using L = ScanLds<DK, NW, E>;
    using V = ElemVec<E>;
    constexpr int KB = M::KB, VEC = L::VEC, DVB = L::DVB, NS = SP::N;
    constexpr int LDQ = L::LDQ, LDT = L::LDT;
    constexpr int NKD = DK / KB, NKC = C / KB, NMT = DK / 16;
    constexpr int NWF = 4 * NKD, NTF = 4 * NKC;
    constexpr int NT = NW * 64;
    constexpr int VPR = DK / VEC;        // 16-byte vectors per q/k row
    constexpr int VPB = DVB / VEC;       // 16-byte vectors per v row block

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    E *sQ = reinterpret_cast<E *>(smem);
    E *sKT = reinterpret_cast<E *>(smem + L::Q);
    E *sVT = reinterpret_cast<E *>(smem + L::Q + L::KT);
    float *sScal = reinterpret_cast<float *>(smem + L::Q + L::KT + L::VT);

    const int i = blockIdx.x, h = blockIdx.y, cb = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n = lane & 15, qd = lane >> 4;
    const int kh = h / (sp.H_v / sp.H_k);
    const int col0 = cb * DVB + 16 * w;
    const E *qg = static_cast<const E *>(sp.q);
    const E *kg = static_cast<const E *>(sp.k);
    const E *vg = static_cast<const E *>(sp.v);
    OT *og = static_cast<OT *>(sp.out);

    // state columns col0..col0+15 in accumulator layout
    floatx4 S[NMT];
    const int sin = sp.state_in ? sp.slot_in[i] : -1;
    if (sin >= 0) {
        const float *base = sp.state_in + (int64_t)sin * sp.slot_stride + (int64_t)h * DK * DV + col0 + n;
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j) S[mt][j] = base[(int64_t)(16 * mt + 4 * qd + j) * DV];
    } else {
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) S[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    const int cs = sp.cstart[i], ce = sp.cstart[i + 1];
    for (int c = cs; c < ce; ++c) {
        const ChunkEntry e = sp.ent[c];
        const int t0 = e.t0, len = e.len;
        const char *blk = sp.blocks + ((size_t)c * sp.H_v + h) * sp.block;
        const char *Wf = blk;
        const char *Tf = blk + NWF * 1024;
        const char *Pf = blk + (NWF + NS * NTF) * 1024;
        const float *scal = reinterpret_cast<const float *>(blk + (NWF + 2 * NS * NTF) * 1024);

        // stage raw Q (row-major), K^T and this block's V^T columns
        for (int vi = tid; vi < C * VPR; vi += NT) {
            const int r = vi / VPR, cv = vi % VPR;
            uint4 kv = make_uint4(0, 0, 0, 0), qv = kv;
            if (r < len) {
                const size_t off = ((size_t)(t0 + r) * sp.H_k + kh) * DK + (size_t)cv * VEC;
                kv = *reinterpret_cast<const uint4 *>(kg + off);
                qv = *reinterpret_cast<const uint4 *>(qg + off);
            }
            *reinterpret_cast<uint4 *>(sQ + r * LDQ + cv * VEC) = qv;
#pragma unroll
            for (int x = 0; x < VEC; ++x) sKT[(cv * VEC + x) * LDT + r] = V::raw(kv, x);
        }
        for (int vi = tid; vi < C * VPB; vi += NT) {
            const int r = vi / VPB, cv = vi % VPB;
            uint4 vv = make_uint4(0, 0, 0, 0);
            if (r < len)
                vv = *reinterpret_cast<const uint4 *>(vg + ((size_t)(t0 + r) * sp.H_v + h) * DV + cb * DVB + cv * VEC);
#pragma unroll
            for (int x = 0; x < VEC; ++x) sVT[(cv * VEC + x) * LDT + r] = V::raw(vv, x);
        }
        for (int x = tid; x < 129; x += NT) sScal[x] = scal[x];
        __syncthreads();

        // the incoming state as two-term B operands, one per dk block
        Frag Sh[NKD], Sl[NKD];
#pragma unroll
        for (int kb = 0; kb < NKD; ++kb) SP::acc(S, kb, 1.f, Sh[kb], Sl[kb]);

        // U = T' V - W S   (token rows, this wave's 16 columns)
        floatx4 U[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            U[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb)
                if (kb * KB <= 16 * rt + 15) {
                    const Frag vb = M::load_rm(sVT + (16 * w + n) * LDT, kb * KB, qd);
                    M::mma(U[rt], load_frag<E>(Tf, rt * NKC + kb, lane), vb);
                    if constexpr (NS == 2) M::mma(U[rt], load_frag<E>(Tf + NTF * 1024, rt * NKC + kb, lane), vb);
                }
#pragma unroll
            for (int kb = 0; kb < NKD; ++kb) {
                const Frag wa = load_frag<E>(Wf, rt * NKD + kb, lane);
                floatx4 t = {0.f, 0.f, 0.f, 0.f};
                M::mma(t, wa, Sh[kb]);
                if constexpr (NS == 2) M::mma(t, wa, Sl[kb]);
                U[rt] -= t;
            }
        }

        // the chunk deltas as two-term B operands (K blocks over tokens)
        Frag Uh[NKC], Ul[NKC];
#pragma unroll
        for (int kb = 0; kb < NKC; ++kb) SP::acc(U, kb, 1.f, Uh[kb], Ul[kb]);

        // O = qs * (Q S) + P U
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            floatx4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKD; ++kb) {
                const Frag qa = M::load_rm(sQ + (16 * rt + n) * LDQ, kb * KB, qd);
                M::mma(O, qa, Sh[kb]);
                if constexpr (NS == 2) M::mma(O, qa, Sl[kb]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) O[j] *= sScal[16 * rt + 4 * qd + j];
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb)
                if (kb * KB <= 16 * rt + 15) {
                    const Frag ph = load_frag<E>(Pf, rt * NKC + kb, lane);
                    M::mma(O, ph, Uh[kb]);
                    if constexpr (NS == 2) {
                        M::mma(O, ph, Ul[kb]);
                        M::mma(O, load_frag<E>(Pf + NTF * 1024, rt * NKC + kb, lane), Uh[kb]);
                    }
                }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * rt + 4 * qd + j;
                if (r < len) og[((size_t)(t0 + r) * sp.H_v + h) * DV + col0 + n] = from_f32<OT>(O[j]);
            }
        }

        // S = gn S + K^T (ks * U)
        const float gn = sScal[128];
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j) S[mt][j] *= gn;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int j = 0; j < 4; ++j) U[rt][j] *= sScal[64 + 16 * rt + 4 * qd + j];
#pragma unroll
        for (int kb = 0; kb < NKC; ++kb) SP::acc(U, kb, 1.f, Uh[kb], Ul[kb]);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb) {
                const Frag ka = M::load_rm(sKT + (16 * mt + n) * LDT, kb * KB, qd);
                M::mma(S[mt], ka, Uh[kb]);
                if constexpr (NS == 2) M::mma(S[mt], ka, Ul[kb]);
            }
        __syncthreads();
    }

    const int sout = sp.slot_out[i];
    if (sout >= 0) {
        float *base = sp.state_out + (int64_t)sout * sp.slot_stride + (int64_t)h * DK * DV + col0 + n;
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j) base[(int64_t)(16 * mt + 4 * qd + j) * DV] = S[mt][j];
    }
}

// --------------------------------------------------------------------------
// launchers
// --------------------------------------------------------------------------
template <typename K>
hipError_t set_lds(K kernel, size_t bytes)
{
    if (bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

struct WsPtrs {
    WsLayout L;
    int32_t *hdr;
    ChunkEntry *ent;
    int32_t *cstart;
    char *blocks;
};

WsPtrs ws_ptrs(const Problem &p, const PrefillArgs &a)
{
    WsPtrs w;
    w.L = ws_layout(p, a.n_seqs, a.total_tokens);
    char *ws = static_cast<char *>(a.workspace);
    w.hdr = reinterpret_cast<int32_t *>(ws);
    w.ent = reinterpret_cast<ChunkEntry *>(ws + w.L.entries);
    w.cstart = reinterpret_cast<int32_t *>(ws + w.L.cstart);
    w.blocks = ws + w.L.blocks;
    return w;
}

template <int DK, typename E>
hipError_t prepare_t(const Problem &p, const PrefillArgs &a, hipStream_t st)
{
    const WsPtrs w = ws_ptrs(p, a);
    hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(1024), 0, st, a.cu_seqlens, a.n_seqs,
                       (int)a.total_tokens, w.L.max_chunks, w.hdr, w.ent, w.cstart);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.total_tokens == 0) return e;
    PrepParams pp{a.q, a.k, a.g, a.beta, w.hdr, w.ent, w.blocks, w.L.block, p.H_k, p.H_v, p.scale, p.eps};
    constexpr size_t lds = PrepLds<DK, E>::BYTES;
    e = set_lds(prep_kernel<DK, E>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prep_kernel<DK, E>), dim3(w.L.max_chunks, p.H_k), dim3(256), lds, st, pp);
    return hipGetLastError();
}

template <int DK, int DV, typename E, typename OT>
hipError_t scan_t(const Problem &p, const PrefillArgs &a, hipStream_t st)
{
    const WsPtrs w = ws_ptrs(p, a);
    constexpr int NW = DV >= 64 ? 4 : DV / 16;
    ScanParams sp{a.q, a.k, a.v, a.state_in, a.state_out, a.out, a.slot_in, a.slot_out, w.cstart,
                  w.ent, w.blocks, w.L.block, p.H_k, p.H_v, p.slot_stride};
    constexpr size_t lds = ScanLds<DK, NW, E>::BYTES;
    hipError_t e = set_lds(scan_kernel<DK, DV, NW, E, OT>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((scan_kernel<DK, DV, NW, E, OT>), dim3(a.n_seqs, p.H_v, DV / (16 * NW)),
                       dim3(NW * 64), lds, st, sp);
    return hipGetLastError();
}

template <int DK>
hipError_t prepare_dk(const Problem &p, const PrefillArgs &a, hipStream_t st)
{
    return p.bf16 ? prepare_t<DK, bf16_t>(p, a, st) : prepare_t<DK, float>(p, a, st);
}

template <int DK, int DV>
hipError_t scan_dv(const Problem &p, const PrefillArgs &a, hipStream_t st)
{
    if (p.bf16)
        return p.out_bf16 ? scan_t<DK, DV, bf16_t, bf16_t>(p, a, st) : scan_t<DK, DV, bf16_t, float>(p, a, st);
    return p.out_bf16 ? scan_t<DK, DV, float, bf16_t>(p, a, st) : scan_t<DK, DV, float, float>(p, a, st);
}

template <int DK>
hipError_t scan_dk(const Problem &p, const PrefillArgs &a, hipStream_t st)
{
    switch (p.d_v) {
    case 32: return scan_dv<DK, 32>(p, a, st);
    case 64: return scan_dv<DK, 64>(p, a, st);
    case 128: return scan_dv<DK, 128>(p, a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t prefill_workspace_bytes(const Problem &p, int32_t n_seqs, int64_t total_tokens)
{
    return ws_layout(p, n_seqs, total_tokens).total;
}

hipError_t launch_prepare(const Problem &p, const PrefillArgs &a, hipStream_t st)
{
    switch (p.d_k) {
    case 32: return prepare_dk<32>(p, a, st);
    case 64: return prepare_dk<64>(p, a, st);
    case 128: return prepare_dk<128>(p, a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_scan(const Problem &p, const PrefillArgs &a, hipStream_t st)
{
    switch (p.d_k) {
    case 32: return scan_dk<32>(p, a, st);
    case 64: return scan_dk<64>(p, a, st);
    case 128: return scan_dk<128>(p, a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
