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
//   2. prep_kernel, one workgroup per (chunk, key head) (eight waves at
//      d_k = d_v = 128), fully parallel:
//      everything that does not depend on the carried state, for all value
//      heads sharing the key head.  K K^T and K Q^T once (bf16 MFMA, fp32
//      accumulate); the decay masks from an fp64 cumulative sum (so
//      exp(G_r - G_c) never forms a factor exp(-G) that would overflow); T by
//      blocked forward substitution in LDS (16x16 diagonal blocks by
//      substitution, off-diagonal blocks with fp32 MFMA); then W, the masked
//      attention P and U0 = T diag(beta) V.  Results go to the workspace as
//      ready-made MFMA operand fragments (W, P, and q / k^T of the key head)
//      and accumulator tiles (U0).
//   3. scan_kernel, one workgroup per (sequence, value head, 16 state
//      columns): walks the sequence's chunks in order with the state in
//      registers for the whole sequence.  Four state waves each take 16
//      token rows of a chunk and own 32 rows of the state; four output
//      waves each take 16 token rows of the output:
//        phase A  state waves:  U = U0 - W S           (token rows)
//                 output waves: Q S                    (token rows)
//        phase B  state waves:  S = gn * S + K^T (ks * U)   (state rows)
//                 output waves: O = qs * (Q S) + P U   (token rows)
//      U and S are exchanged through LDS as ready-made operand fragments;
//      each wave loads its own operands from the workspace straight into
//      registers, one chunk ahead.  With the layer prologue the launch that
//      holds a sequence's last chunk also writes its new convolution state.
//
// Norms, scale, beta and decay are folded into per-row / per-column scalars
// of raw (bf16) operands, so the inputs are used as MFMA operands exactly as
// stored.  A final partial chunk is zero-padded; padded rows carry beta = 0,
// g = 0 and zero norms, which makes them the identity on the state.
#include <atomic>

#include "../../include/gdn.h"
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

constexpr int C = kChunk;

struct ChunkEntry {
    int32_t seq, t0, len, first;   // first: the sequence's first chunk
};

// --------------------------------------------------------------------------
// workspace geometry
//
// per (chunk, value head), in 1 KiB units:
//   W fragments (4 x NKD) | [W lo (4 x NKD)] | P hi (4 x NKC) | [P lo (4 x NKC)] | scalars | U0 tiles (4 x NCT)
// per (chunk, key head):
//   q fragments (4 x NKD) | [q lo (4 x NKD)] | k^T fragments (NMT x NKC) | [k^T lo (NMT x NKC)]
// (the lo parts exist when q and k are two-term operands, see prep_kernel)
// A fragment is a 16-row x KB-deep MFMA operand, 64 lanes x 16 bytes.  The
// scalars are qs[64] (q scale * e^{G_r}), ks[64] (e^{G_n - G_r} / |k_r|), gn,
// and the chunk's first token and length (int bits).  U0 tiles are stored
// column-tile major (ct, rt) so a workgroup's column tiles are contiguous.
// --------------------------------------------------------------------------
__host__ __device__ constexpr int kb_of(bool bf16) { return bf16 ? 32 : 16; }
__host__ __device__ constexpr int ns_of(bool bf16) { return bf16 ? 2 : 1; }
__host__ __device__ constexpr int vshared_kib(int dk, bool bf16, bool si) {
    return (si ? 2 : 1) * 4 * (dk / kb_of(bf16)) + ns_of(bf16) * 4 * (C / kb_of(bf16)) + 1;
}
__host__ __device__ constexpr int vblk_kib(int dk, int dv, bool bf16, bool si) {
    return vshared_kib(dk, bf16, si) + 4 * (dv / 16);
}
__host__ __device__ constexpr int kblk_kib(int dk, bool bf16, bool si) {
    return (si ? 2 : 1) * (4 * (dk / kb_of(bf16)) + (dk / 16) * (C / kb_of(bf16)));
}

// SI: q and k enter the scan as two-term (hi + lo) bf16 operands
template <int DK, int DV, typename E, bool SI = false> struct Geo {
    using M = Mfma<E>;
    static constexpr bool BF = sizeof(E) == 2;
    static constexpr int KB = M::KB, TPB = M::TPB, NS = Split<E>::N;
    static constexpr int NKD = DK / KB, NKC = C / KB, NMT = DK / 16, NCT = DV / 16;
    static constexpr int NWF = 4 * NKD, NPF = 4 * NKC, NQF = 4 * NKD, NKF = NMT * NKC;
    static constexpr int NQS = SI ? 2 : 1;
    static constexpr int F_W = 0, F_WL = NWF, F_PH = NQS * NWF, F_PL = F_PH + NPF, F_SCAL = F_PH + NS * NPF;
    static constexpr int SV = F_SCAL + 1;                 // shared part of the value-head block
    static constexpr int F_U0 = SV;
    static constexpr int VBLK = SV + 4 * NCT;
    static constexpr int F_Q = 0, F_QL = NQF, F_KT = NQS * NQF, F_KTL = F_KT + NKF;
    static constexpr int KBLK = NQS * (NQF + NKF);
    static_assert(!SI || BF, "two-term q and k are bf16 operands");
    static_assert(VBLK == vblk_kib(DK, DV, BF, SI) && KBLK == kblk_kib(DK, BF, SI), "geometry");
};

struct WsLayout {
    size_t entries, cstart, vblocks, kblocks, vblk, kblk, obuf, carry, total;
    int max_chunks;
};

// With the epilogue and a bf16 output, the scan's fp32 o is staged in the
// workspace so that the result is rounded once.
bool stage_o(const Problem &p) { return p.z && p.out_bf16; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Compute units of the current device (cached per device).
int cu_count()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Operand type of the chunked form: that of the inputs.  With the
// convolution prologue and bf16 rows, q, k, v become two-term bf16 operands
// (see prep_kernel).
bool op_bf16(const Problem &p) { return p.bf16 != 0; }
bool op_split(const Problem &p) { return p.bf16 && p.conv_w; }

int chunk_count(int32_t n_seqs, int64_t T)
{
    return n_seqs == 1 ? (int)((T + C - 1) / C) : (int)max_chunks(n_seqs, T);
}

// slots: WY-factor slots (chunks held at once); 0 or more than the batch has
// means one per chunk.  With fewer slots than chunks the batch runs as
// several ranges, and two carry states pass a sequence's state from range to
// range.
WsLayout ws_layout(const Problem &p, int32_t n_seqs, int64_t T, int slots)
{
    WsLayout L;
    const bool bf = op_bf16(p);
    L.max_chunks = (int)max_chunks(n_seqs, T);
    const size_t fs = slots > 0 && slots < L.max_chunks ? (size_t)slots : (size_t)L.max_chunks;
    L.entries = 256;
    L.cstart = align256(L.entries + sizeof(ChunkEntry) * (size_t)L.max_chunks);
    L.vblocks = align256(L.cstart + sizeof(int32_t) * ((size_t)n_seqs + 1));
    L.vblk = (size_t)vblk_kib(p.d_k, p.d_v, bf, op_split(p)) * 1024;
    L.kblk = (size_t)kblk_kib(p.d_k, bf, op_split(p)) * 1024;
    L.kblocks = L.vblocks + L.vblk * fs * p.H_v;
    L.obuf = align256(L.kblocks + L.kblk * fs * p.H_k);
    L.carry = align256(L.obuf + (stage_o(p) ? sizeof(float) * (size_t)T * p.H_v * p.d_v : 0));
    const bool ranges = slots > 0 && slots < chunk_count(n_seqs, T);
    L.total = L.carry + (ranges ? 2 * sizeof(float) * (size_t)p.H_v * p.d_k * p.d_v : 0);
    return L;
}

// --------------------------------------------------------------------------
// 1. chunk table
// --------------------------------------------------------------------------
constexpr int kTableSeqsInLds = 4096;

__global__ __launch_bounds__(1024) void chunk_table_kernel(
    const int32_t *__restrict__ cu, int n_seqs, int T, int max_ch,
    int32_t *__restrict__ hdr, ChunkEntry *__restrict__ ent, int32_t *__restrict__ cstart)
{
    __shared__ int wsum[16];
    __shared__ int s_carry;
    __shared__ int s_cs[kTableSeqsInLds + 1];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const bool small = n_seqs <= kTableSeqsInLds;
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
            if (small) {
                s_cs[i] = start;
            } else {
                for (int c = 0; c < nc; ++c) {
                    const int idx = start + c;
                    if (idx < max_ch) ent[idx] = ChunkEntry{i, tb + c * C, min(C, te - tb - c * C), c == 0};
                }
            }
        }
        __syncthreads();
        if (tid == 0) s_carry = carry + total;
        __syncthreads();
    }
    const int n = min(s_carry, max_ch);
    if (tid == 0) {
        cstart[n_seqs] = n;
        hdr[0] = n;
        if (small) s_cs[n_seqs] = s_carry;
    }
    if (!small) return;
    __syncthreads();
    // one thread per chunk: binary search for the owning sequence
    for (int j = tid; j < n; j += 1024) {
        int lo = 0, hi = n_seqs - 1;
        while (lo < hi) {                       // last i with s_cs[i] <= j
            const int mid = (lo + hi + 1) >> 1;
            if (s_cs[mid] <= j) lo = mid; else hi = mid - 1;
        }
        const int tb = min(max(cu[lo], 0), T);
        const int te = min(max(cu[lo + 1], tb), T);
        const int c = j - s_cs[lo];
        ent[j] = ChunkEntry{lo, tb + c * C, min(C, te - tb - c * C), c == 0};
    }
}

// --------------------------------------------------------------------------
// helpers
// --------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 v = {(__bf16)a, (__bf16)b};      // v_cvt_pk_bf16_f32, round to nearest even
    return __builtin_bit_cast(uint32_t, v);
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
    bf16x4 h, l;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        h[j] = (__bf16)v[j];
        l[j] = (__bf16)(v[j] - (float)h[j]);
    }
    const size_t off = ((size_t)f * 64 + lane) * 16 + half * 8;
    *reinterpret_cast<bf16x4 *>(reinterpret_cast<char *>(hi_base) + off) = h;
    *reinterpret_cast<bf16x4 *>(reinterpret_cast<char *>(lo_base) + off) = l;
}
template <> __device__ __forceinline__ void store_quarter2<float>(void *hi_base, void *lo_base, int f, int lane, int half, floatx4 v) {
    (void)lo_base;
    store_quarter<float>(hi_base, f, lane, half, v);
}

// Both halves of fragment f at once (bf16 operands: two 16-column tiles of
// a 32-deep K block, v0 the first), one 16-byte store per lane: written half
// by half, each store instruction would fill only half of the lines it
// touches.  Single-term, and two-term into hi_base / lo_base.
__device__ __forceinline__ void store_pair(void *base, int f, int lane, floatx4 v0, floatx4 v1) {
    const uint4 u = make_uint4(pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]), pack_bf16x2(v1[0], v1[1]),
                               pack_bf16x2(v1[2], v1[3]));
    *reinterpret_cast<uint4 *>(reinterpret_cast<char *>(base) + ((size_t)f * 64 + lane) * 16) = u;
}
__device__ __forceinline__ void store_pair2(void *hi_base, void *lo_base, int f, int lane, floatx4 v0, floatx4 v1) {
    floatx4 h0, h1, l0, l1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        h0[j] = (float)(__bf16)v0[j];
        h1[j] = (float)(__bf16)v1[j];
        l0[j] = v0[j] - h0[j];
        l1[j] = v1[j] - h1[j];
    }
    store_pair(hi_base, f, lane, h0, h1);
    store_pair(lo_base, f, lane, l0, l1);
}

// 16 bytes of an input row (q, k, v or the mixed rows), which the preparation
// reads once.  The load is non-temporal, so a miss does not allocate the line
// in the MALL (the memory-side last-level cache): that cache then holds the
// WY factors the preparation writes until the scan reads them back.  With
// ordinary loads the input rows took part of it, and the scan after a
// 4096-token preparation ran 78-80 us instead of the 62-64 us it takes on
// cached factors.
__device__ __forceinline__ u32x4 load_once(const bf16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ u32x4 load_once(const float *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// Squared norm of the 16 bytes a lane loaded from a q / k row.
template <typename E> __device__ __forceinline__ float sumsq16(u32x4 u);
template <> __device__ __forceinline__ float sumsq16<bf16_t>(u32x4 u) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float a = __uint_as_float(u[e] << 16), b = __uint_as_float(u[e] & 0xffff0000u);
        s += a * a + b * b;
    }
    return s;
}
template <> __device__ __forceinline__ float sumsq16<float>(u32x4 u) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) s += __uint_as_float(u[e]) * __uint_as_float(u[e]);
    return s;
}

// Operand fragment read transposed out of a row-major LDS matrix X[k][n]
// (leading dimension ld elements): lane (qd, n) receives X[k0 + 4qd + j][n0 + n]
// (and, for bf16, X[k0 + 16 + 4qd + j][n0 + n]), j = 0..3.  That is the B
// operand of a K block whose K index runs over X's rows, and equally the A
// operand of X^T.  For bf16 the transpose is done by ds_read_b64_tr_b16: in
// each group of 16 lanes, lane i receives element i % 4 of the 8-byte words
// fetched by lanes i / 4 + 4j, so lane p of group qd fetches row
// k0 + 4qd + p / 4, columns n0 + 4 (p % 4) .. +3.
template <typename E> struct TrLoad;
template <> struct TrLoad<bf16_t> {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    __device__ static __forceinline__ bf16x8 frag(const bf16_t *X, int ld, int k0, int n0, int lane) {
        const int qd = lane >> 4, p = lane & 15;
        const bf16_t *a = X + (k0 + 4 * qd + (p >> 2)) * ld + n0 + 4 * (p & 3);
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(void *)(a));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(void *)(a + 16 * ld));
        const v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8, v);
    }
};
template <> struct TrLoad<float> {
    __device__ static __forceinline__ floatx4 frag(const float *X, int ld, int k0, int n0, int lane) {
        const int qd = lane >> 4, n = lane & 15;
        floatx4 f;
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] = X[(k0 + 4 * qd + j) * ld + n0 + n];
        return f;
    }
};

// e^d for d = G_r - G_c <= 0 given in fp64: the difference is scaled to
// base 2 in fp64 and rounded once to fp32 for v_exp_f32 (about 1 ulp; the
// result underflows to 0 for d below about -103).
__device__ __forceinline__ float exp_neg(double d) {
    return __builtin_amdgcn_exp2f((float)(d * 1.4426950408889634));
}

// A DPP move of an fp64 value (both halves; lanes without a source, and
// rows outside RM, read zero).  CTRL 0x111..0x118: row_shr 1..8 (within rows
// of 16 lanes); 0x142: row_bcast 15 (lane 15 of each row to the next row);
// 0x143: row_bcast 31 (lane 31 to rows 2 and 3).
template <int CTRL, int RM> __device__ __forceinline__ double dpp_f64(double x) {
    const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, RM, 0xf, true);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, RM, 0xf, true);
    return __builtin_bit_cast(double, ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo);
}
// Inclusive prefix sum of an fp64 value over the 64 lanes of a wave: within
// each row of 16 lanes by row shifts, then across rows by the broadcasts of
// lanes 15 and 31.  The moves run in the vector ALU, without the LDS round
// trip of a shuffle.
__device__ __forceinline__ double wave_inclusive_sum(double x) {
    x += dpp_f64<0x111, 0xf>(x);
    x += dpp_f64<0x112, 0xf>(x);
    x += dpp_f64<0x114, 0xf>(x);
    x += dpp_f64<0x118, 0xf>(x);
    x += dpp_f64<0x142, 0xa>(x);
    x += dpp_f64<0x143, 0xc>(x);
    return x;
}
__device__ __forceinline__ double readlane_f64(double x, int l) {
    const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}

// The 10 lower 16x16 tile pairs (rt, ct), ct <= rt, of a 64x64 matrix in
// row order, and the 6 strictly upper ones.  Computed, not tabulated: a table
// indexed per wave becomes a vector memory load, and on gfx9 waiting for it
// also waits for every store issued before it.
__device__ __forceinline__ int low_r(int it) { return it >= 6 ? 3 : it >= 3 ? 2 : it >= 1 ? 1 : 0; }
__device__ __forceinline__ int low_c(int it) { const int r = low_r(it); return it - r * (r + 1) / 2; }
__device__ __forceinline__ int up_r(int z) { return z >= 5 ? 2 : z >= 3 ? 1 : 0; }
__device__ __forceinline__ int up_c(int z) { const int r = up_r(z); return r == 0 ? z + 1 : r == 1 ? z - 1 : 3; }

// Product tile of slot s in wave w of the preparation (0..9: the lower
// tiles of K K^T, 10..19: the tiles of K Q^T; -1: none).  Four waves: w + 4 s.
// Eight waves: the A tiles w and, in waves 0 and 1, 8 + w; the P tiles in the
// pairs that fill one bf16 operand fragment (the two 16-column halves of a
// 32-deep K block): waves 2..5 the tiles 1+2, 3+4, 6+7 and 8+9, waves 0 and
// 1 the tiles 0 and 5 ((0,0) and (2,2)), whose partners lie above the
// diagonal and are zero.
template <int NW> __device__ __forceinline__ int prod_it(int w, int s)
{
    if constexpr (NW == 4) {
        return w + 4 * s;
    } else {
        if (s == 0) return w;
        if (w < 2) return s == 1 ? 8 + w : (w == 0 ? 10 : 15);
        if (w < 6) return 10 + (w == 2 ? 1 : w == 3 ? 3 : w == 4 ? 6 : 8) + (s - 1);
        return -1;
    }
}

struct PrepParams {
    const void *q, *k, *v;
    const float *g, *beta;
    const int32_t *hdr;
    const ChunkEntry *ent;
    char *vblocks, *kblocks;
    int H_k, H_v;
    float scale, eps;
    int single_T;      // >= 0: one sequence of this many tokens, no chunk table
    Gates gates;       // raw gate projections, or g and beta as given
    int64_t rs_qk, rs_v;       // row strides (elements) of q / k and of v
    // convolution prologue (prep_kernel<..., true>): q, k, v are channel
    // ranges of the mixed rows; conv_in holds the slot rows (convolution state
    // first), or any readable buffer when has_state is 0
    const float *conv_w;
    const float *conv_in;
    const int32_t *slot_in;
    int64_t slot_stride;
    int has_state;
    // 1: one workgroup per (chunk, value head) instead of per (chunk, key
    // head), for grids too small to fill the GPU (K K^T is then formed once
    // per value head)
    int head_split;
    int chunk_base;    // blockIdx.x = 0 is this chunk of the batch; its factors go to slot 0
    // debug record (null: off): G, T and W of the chunk holding packed token
    // dbg_t, for value head dbg_h
    gdn_debug_chunk *dbg = nullptr;
    int dbg_t = -1, dbg_h = -1;
};

// LDS of the preparation kernel.  Rows are padded so that the row stride is
// 8 banks (mod 64): the transposed reads (4 rows x 32 bytes per 16 lanes) and
// the row reads of 16 different rows then hit distinct banks.
// SI: the lo parts of two-term K and Q / V rows follow.
template <int DK, int DV, typename E, bool SI = false> struct PrepLds {
    static constexpr int PAD = sizeof(E) == 2 ? 16 : 4;
    static constexpr int LDK = DK + PAD;                  // K rows
    static constexpr int DX = DK > DV ? DK : DV;
    static constexpr int LDX = DX + PAD;                  // Q rows, then V rows of one value head
    static constexpr int LDA = C + 4;                     // A and T (fp32)
    static constexpr size_t OFF_K = 0;
    static constexpr size_t OFF_X = OFF_K + (size_t)C * LDK * sizeof(E);
    static constexpr size_t OFF_A = OFF_X + (size_t)C * LDX * sizeof(E);
    static constexpr size_t OFF_T = OFF_A + (size_t)C * LDA * sizeof(float);
    static constexpr size_t OFF_G = OFF_T + (size_t)C * LDA * sizeof(float);
    static constexpr int NH = 4;                          // value heads whose row scalars are held at once
    static constexpr size_t OFF_S = OFF_G + NH * C * sizeof(double);
    static constexpr size_t OFF_KL = OFF_S + (2 + 3 * NH) * C * sizeof(float);
    static constexpr size_t OFF_XL = OFF_KL + (SI ? (size_t)C * LDK * sizeof(E) : 0);
    static constexpr size_t BYTES = OFF_XL + (SI ? (size_t)C * LDX * sizeof(E) : 0);
};

// --------------------------------------------------------------------------
// 2. per-chunk preparation (state independent)
// --------------------------------------------------------------------------
// silu of a 4-tap causal convolution, per channel: x0 oldest, x3 current.
__device__ __forceinline__ float conv_silu4(float4 w, float x0, float x1, float x2, float x3)
{
    return silu(w.x * x0 + w.y * x1 + w.z * x2 + w.w * x3);
}

// Raw fp32 bits of one element of E through a buffer resource (zero past the
// range's end).
template <typename E> __device__ __forceinline__ uint32_t buf_bits(__amdgpu_buffer_rsrc_t r, uint32_t off);
template <> __device__ __forceinline__ uint32_t buf_bits<bf16_t>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0) << 16;
}
template <> __device__ __forceinline__ uint32_t buf_bits<float>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// The VEC values of a 16-byte vector as fp32, and back (rounded to E).
template <typename E> __device__ __forceinline__ void unpack16(u32x4 u, float *f);
template <> __device__ __forceinline__ void unpack16<bf16_t>(u32x4 u, float *f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = __uint_as_float(u[e] << 16);
        f[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
    }
}
template <> __device__ __forceinline__ void unpack16<float>(u32x4 u, float *f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(u[e]);
}
template <typename E> __device__ __forceinline__ u32x4 pack16(const float *f);
template <> __device__ __forceinline__ u32x4 pack16<bf16_t>(const float *f) {
    return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                 pack_bf16x2(f[6], f[7])};
}
template <> __device__ __forceinline__ u32x4 pack16<float>(const float *f) {
    return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
}

// silu(conv) of NR consecutive rows row0.. of one 16-byte column vector (VEC
// channels), from raw[0 .. NR+2] holding rows row0-3 .. row0+NR-1; rows
// before the chunk (negative) come from the LDS history hist[m][.] (m = row +
// 3, fp32) at column offset hoff, the taps from w[e] (channel e).  Results are
// zero from row `len` on; with a lo array they are stored two-term (hi =
// rounded to E, lo = the remainder rounded to E), else rounded once.
template <typename E, int NR>
__device__ __forceinline__ void conv_rows(const u32x4 *raw, const float4 *w, int row0, int len, const float *hist,
                                          int hld, int hoff, u32x4 *hi, u32x4 *lo)
{
    constexpr int VEC = 16 / (int)sizeof(E);
#pragma unroll
    for (int p = 0; p < NR; ++p) {
        float x[4][VEC];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            unpack16<E>(raw[p + j], x[j]);
            if (row0 - 3 + p + j < 0) {
                const float *hp = hist + (row0 + p + j) * hld + hoff;
#pragma unroll
                for (int e = 0; e < VEC; e += 4) {
                    const float4 h4 = *reinterpret_cast<const float4 *>(hp + e);
                    x[j][e] = h4.x; x[j][e + 1] = h4.y; x[j][e + 2] = h4.z; x[j][e + 3] = h4.w;
                }
            }
        }
        float y[VEC], r[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) y[e] = conv_silu4(w[e], x[0][e], x[1][e], x[2][e], x[3][e]);
        const bool live = row0 + p < len;
        const u32x4 h = pack16<E>(y);
        hi[p] = live ? h : u32x4{0u, 0u, 0u, 0u};
        if (lo) {
            float hf[VEC];
            unpack16<E>(h, hf);
#pragma unroll
            for (int e = 0; e < VEC; ++e) r[e] = y[e] - hf[e];
            lo[p] = live ? pack16<E>(r) : u32x4{0u, 0u, 0u, 0u};
        }
    }
}

// CONV: the convolution prologue (build_layer_attn_linear_core on the page
// "ik_llama.cpp src/llama-delta-net.cpp": ggml_ssm_conv + ggml_silu) is formed
// while the rows are loaded.  A thread then owns KL (VL) consecutive rows of
// one 16-byte column vector; the three rows before a thread's first are
// loaded too (K, Q) or read back from LDS (V), and the three rows before the
// chunk (the slot's convolution state for a sequence's first chunk, else the
// preceding rows) are staged through LDS with the taps of V.  After SiLU the
// keys of neighbouring tokens are correlated and a single bf16 rounding of q,
// k or v moves the result by several percent of its rms, so with bf16 rows
// the convolution output becomes two-term bf16 operands (SI: hi + lo, about
// 16 significant bits) in every product that reads q, k or v, and with fp32
// rows the operands stay fp32.
template <int DK, int DV, typename E, bool CONV, int NW>
__global__ __launch_bounds__(64 * NW, ((sizeof(E) == 2 && !CONV) ? 2 : 1) * NW / 4) void prep_kernel(PrepParams pp)
{
    constexpr bool SI = CONV && sizeof(E) == 2;
    using M = Mfma<E>;
    using SP = Split<E>;
    using G = Geo<DK, DV, E, SI>;
    using L = PrepLds<DK, DV, E, SI>;
    using TR = TrLoad<E>;
    using Frag = typename M::Frag;
    constexpr int KB = M::KB, TPB = M::TPB, NS = SP::N;
    constexpr int VEC = 16 / (int)sizeof(E);
    constexpr int LDK = L::LDK, LDX = L::LDX, LDA = L::LDA;
    constexpr int NKD = G::NKD, NKC = G::NKC, NMT = DK / 16, NCT = DV / 16;
    constexpr int VPR = DK / VEC;         // 16-byte vectors per q/k row
    constexpr int VPRV = DV / VEC;        // 16-byte vectors per v row
    constexpr int NT = 64 * NW;           // threads (NW = 4 or 8 waves)
    static_assert(NW == 4 || NW == 8, "four or eight waves");

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    E *sK = reinterpret_cast<E *>(smem + L::OFF_K);
    E *sX = reinterpret_cast<E *>(smem + L::OFF_X);
    float *sA = reinterpret_cast<float *>(smem + L::OFF_A);
    float *sT = reinterpret_cast<float *>(smem + L::OFF_T);
    E *sKL = reinterpret_cast<E *>(smem + L::OFF_KL);           // SI: lo parts of K
    E *sXL = reinterpret_cast<E *>(smem + L::OFF_XL);           //     and of Q / V
    constexpr int NH = L::NH;
    double *sGh = reinterpret_cast<double *>(smem + L::OFF_G);  // [NH][C] G_r = cumsum of g
    float *sRK = reinterpret_cast<float *>(smem + L::OFF_S);    // 1 / |k_r|
    float *sRQ = sRK + C;                                       // scale / |q_r|
    float *sRAh = sRQ + C;                                      // [NH][C] beta_r / |k_r|  (rows of A)
    float *sBetah = sRAh + NH * C;                              // [NH][C] beta_c          (columns of T for U0)
    float *sColh = sBetah + NH * C;                             // [NH][C] beta_c e^{G_c} / |k_c|  (columns of T for W)

    const int chunk = blockIdx.x + pp.chunk_base;
    const int slot = blockIdx.x;     // its factors' place in the workspace (relative to the range)
    const int ratio = pp.H_v / pp.H_k;
    const int kh = pp.head_split ? blockIdx.y / ratio : blockIdx.y;
    // value heads of this workgroup: [jbeg, jend) of the key head's ratio;
    // row scalars are computed for NH heads at a time from jbase on
    const int jbeg = pp.head_split ? blockIdx.y % ratio : 0;
    const int jend = pp.head_split ? jbeg + 1 : ratio;
    int t0, len, seq, first;
    if (pp.single_T >= 0) {
        // a single sequence covers tokens [0, T): chunk c is [64c, min(64c + 64, T))
        if (chunk * C >= pp.single_T) return;
        t0 = chunk * C;
        len = min(C, pp.single_T - t0);
        seq = 0;
        first = chunk == 0;
    } else {
        if (chunk >= pp.hdr[0]) return;
        const ChunkEntry ce = pp.ent[chunk];
        t0 = ce.t0;
        len = ce.len;
        seq = ce.seq;
        first = ce.first;
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = w % NH;                 // waves NH.. repeat the scalars of waves 0..NH-1
    const int n = lane & 15, qd = lane >> 4;
    const E *qg = static_cast<const E *>(pp.q);
    const E *kg = static_cast<const E *>(pp.k);
    const E *vg = static_cast<const E *>(pp.v);

    // g and beta of up to NH value heads (wave w: head j0 + w mod NH, lane: row)
    // Loads here are unconditional (clamped row / head, zero selected
    // afterwards): a load inside a branch leaves the compiler unable to count
    // outstanding memory operations, and the next wait for it then also waits
    // for every store issued before.  A wave past the last head repeats the
    // last one (identical values written twice).
    // The raw gate activations are applied in head_scalars, where the values
    // are used: applied here, they would make the loads' first wait a wait
    // for every load issued before them.
    float gq = 0.f, bq = 0.f, grate = 0.f, gbias = 0.f;
    const int lrow = min(lane, len - 1);
    auto load_gb = [&](int j0) {
        const int hh = kh * ratio + min(j0 + wn, ratio - 1);
        gq = pp.g[(size_t)(t0 + lrow) * pp.H_v + hh];
        bq = pp.beta[(size_t)(t0 + lrow) * pp.H_v + hh];
        grate = pp.gates.rate[hh];
        gbias = pp.gates.bias[hh];
    };
    // cumulative log-decay (fp64) and the per-row scalars of those heads
    auto head_scalars = [&](int j0) {
        const int jw = min(j0 + wn, ratio - 1);
        const int hh = kh * ratio + jw, hs = jw % NH;
        float *scal = reinterpret_cast<float *>(pp.vblocks + ((size_t)slot * pp.H_v + hh) * ((size_t)G::VBLK * 1024) +
                                                G::F_SCAL * 1024);
        const int r = lane;
        const float gl = pp.gates.raw ? gate_g(gq, gbias, grate) : gq;
        const float bl = pp.gates.raw ? gate_beta(bq) : bq;
        const float gv = lane < len ? gl : 0.f;
        const float bv = lane < len ? bl : 0.f;
        const double Gc = wave_inclusive_sum((double)gv);
        const double Gn = readlane_f64(Gc, 63);
        const float rk = sRK[r];
        const float eG = expf((float)Gc);
        sGh[hs * C + r] = Gc;
        sRAh[hs * C + r] = bv * rk;
        sBetah[hs * C + r] = bv;
        sColh[hs * C + r] = bv * eG * rk;
        scal[r] = sRQ[r] * eG;                              // qs: q scale * e^{G_r}
        scal[64 + r] = rk * expf((float)(Gn - Gc));         // ks: e^{G_n - G_r} / |k_r|
        // gn = e^{G_n}, the chunk's first token and length (int bits): lanes
        // 0..2; the others fall outside the 12-byte buffer and are dropped
        const float tail = lane == 0 ? expf((float)Gn) : __int_as_float(lane == 1 ? t0 : len);
        buffer_store(tail, raw_buffer(scal + 128, 12), (uint32_t)lane * 4u);
    };
    // prologue: the slot holding this sequence's convolution state (row 0 of
    // a readable buffer when there is none; its values are then not used)
    int cslot = 0;
    bool state_ok = false;
    if constexpr (CONV) {
        const int s_in = pp.slot_in[seq];
        state_ok = pp.has_state && s_in >= 0;
        cslot = state_ok ? s_in : 0;
    }
    // the slot's stored convolution inputs, read only for a sequence's first
    // chunk (an empty range otherwise, and without a state)
    const auto hs = raw_buffer(const_cast<float *>(pp.conv_in) + (size_t)cslot * pp.slot_stride,
                               CONV && first && state_ok ? (uint32_t)(2 * pp.H_k * DK + pp.H_v * DV) * 12u : 0u);
    const size_t vch0 = 2 * (size_t)pp.H_k * DK;          // first v channel of the mixed rows

    // V rows of one value head, loaded one head ahead into registers (with
    // the prologue: the thread's VL consecutive rows and its share of the
    // head's three history rows and of its taps, both staged through LDS;
    // the three rows before a thread's first are read back from LDS once
    // every row is there)
    constexpr int VL = (C * VPRV + NT - 1) / NT;
    constexpr int NHV = CONV ? (3 * DV + NT - 1) / NT : 1;
    constexpr int NWV = CONV ? (4 * DV + NT - 1) / NT : 1;
    u32x4 vpre[VL];
    float vh[NHV], vw[NWV];
    const int vrow0 = (tid / VPRV) * VL, vcv = tid % VPRV;
    static_assert(C * VPRV % NT == 0 && C * VPR % NT == 0, "whole vectors per thread");
    // When the rows are not needed (the prefetch after the last head) every
    // lane reads the head's first 16 bytes instead: the loads still issue, so
    // every wait counts exactly, but together they read one line (a reload of
    // the last head's rows added 16 MiB of reads to a 4096-token call).
    auto load_v = [&](int hh, bool live) {
        const E *v0 = vg + (size_t)t0 * pp.rs_v + (size_t)hh * DV;
        if constexpr (!CONV) {
#pragma unroll
            for (int p = 0; p < VL; ++p) {
                const int vi = tid + NT * p;
                const int r = vi / VPRV, cv = vi % VPRV;
                const u32x4 x = load_once(live ? v0 + (size_t)min(r, len - 1) * pp.rs_v + cv * VEC : v0);
                vpre[p] = r < len ? x : u32x4{0u, 0u, 0u, 0u};
            }
        } else {
#pragma unroll
            for (int p = 0; p < VL; ++p) {
                const int rr = min(vrow0 + p, len - 1);
                vpre[p] = load_once(live ? v0 + (size_t)rr * pp.rs_v + vcv * VEC : v0);
            }
            // history: the three rows before the chunk, or for a sequence's
            // first chunk the slot's stored inputs (see the K and Q history)
            const auto hr = raw_buffer(const_cast<E *>(vg) + (first ? 0 : (size_t)(t0 - 3) * pp.rs_v),
                                       first ? 0u : 3u * (uint32_t)pp.rs_v * (uint32_t)sizeof(E));
#pragma unroll
            for (int j = 0; j < NHV; ++j) {
                const int idx = min(tid + NT * j, 3 * DV - 1);
                const int m = idx / DV, c = idx % DV;
                const uint32_t br = buf_bits<E>(hr, (uint32_t)((size_t)m * pp.rs_v + (size_t)hh * DV + c) * sizeof(E));
                const uint32_t bs = __builtin_amdgcn_raw_buffer_load_b32(
                    hs, (uint32_t)((vch0 + (size_t)hh * DV + c) * 3 + m) * 4u, 0, 0);
                vh[j] = __uint_as_float(br | bs);
            }
#pragma unroll
            for (int j = 0; j < NWV; ++j)
                vw[j] = pp.conv_w[(vch0 + (size_t)hh * DV) * 4 + min(tid + NT * j, 4 * DV - 1)];
        }
    };


    // 1. K and Q rows of the chunk (row-major, zero past the end) and their
    //    inverse norms; a row's VPR vectors sit in VPR adjacent lanes
    constexpr int KL = C * VPR / NT;      // 16-byte vectors of K (and of Q) per thread
    constexpr int KR = CONV ? KL + 3 : KL;
    constexpr int NHK = CONV ? (6 * DK + NT - 1) / NT : 1;
    const int krow0 = (tid / VPR) * KL, kcv = tid % VPR;
    u32x4 kx[KL], qx[KL], kxl[SI ? KL : 1], qxl[SI ? KL : 1];
    u32x4 kraw[CONV ? KR : 1], qraw[CONV ? KR : 1];
    float hk[NHK];
    float4 wt = make_float4(0.f, 0.f, 0.f, 0.f);   // CONV: this thread's float4 of the key head's taps
    if constexpr (!CONV) {
#pragma unroll
        for (int p = 0; p < KL; ++p) {
            const int vi = tid + NT * p;
            const int r = vi / VPR, cv = vi % VPR;
            const size_t off = (size_t)(t0 + min(r, len - 1)) * pp.rs_qk + (size_t)kh * DK + (size_t)cv * VEC;
            kx[p] = load_once(kg + off);
            qx[p] = load_once(qg + off);
        }
    } else {
#pragma unroll
        for (int u = 0; u < KR; ++u) {
            const int rr = min(max(krow0 - 3 + u, 0), len - 1);
            const size_t off = (size_t)(t0 + rr) * pp.rs_qk + (size_t)kh * DK + (size_t)kcv * VEC;
            kraw[u] = load_once(kg + off);
            qraw[u] = load_once(qg + off);
        }
        // three history rows of the key head's q and k channels, [m][q | k]:
        // the rows before the chunk, or for a sequence's first chunk the
        // slot's stored inputs (zero without a state).  Each is read through a
        // buffer range that is empty when it does not apply (reads as zero
        // bits) and the raw bits are or-ed: a select between two loads on a
        // uniform condition is compiled into a branch around each load, and
        // each branch then ends in a wait for every load issued before it.
        const uint32_t rbytes = first ? 0u : 3u * (uint32_t)pp.rs_qk * (uint32_t)sizeof(E);
        const size_t rrow = first ? 0 : (size_t)(t0 - 3) * pp.rs_qk;
        const auto hq = raw_buffer(const_cast<E *>(qg) + rrow, rbytes);
        const auto hkb = raw_buffer(const_cast<E *>(kg) + rrow, rbytes);
#pragma unroll
        for (int j = 0; j < NHK; ++j) {
            const int idx = min(tid + NT * j, 6 * DK - 1);
            const int m = idx / (2 * DK), c2 = idx % (2 * DK);
            const bool isk = c2 >= DK;
            const int c = isk ? c2 - DK : c2;
            const uint32_t ro = (uint32_t)((size_t)m * pp.rs_qk + (size_t)kh * DK + c) * sizeof(E);
            const uint32_t bq = buf_bits<E>(hq, isk ? kDropOffset : ro);
            const uint32_t bk = buf_bits<E>(hkb, isk ? ro : kDropOffset);
            const size_t ch = (isk ? (size_t)pp.H_k * DK : 0) + (size_t)kh * DK + c;
            const uint32_t bs = __builtin_amdgcn_raw_buffer_load_b32(hs, (uint32_t)(ch * 3 + m) * 4u, 0, 0);
            hk[j] = __uint_as_float(bq | bk | bs);
        }
        // the taps of the key head's q and k channels ([q | k] x 4, 4 KiB at
        // DK = 128), one float4 per thread and staged through LDS: every row
        // group needs all of them, and loaded per thread they would move 16
        // times those bytes through the CU's load path
        {
            const int tt = min(tid, 2 * DK - 1);
            const size_t ch = (tt < DK ? 0 : (size_t)pp.H_k * DK - DK) + (size_t)kh * DK + tt;
            wt = *reinterpret_cast<const float4 *>(pp.conv_w + ch * 4);
        }
    }
    // the first value heads' g and beta: issued after K and Q (the
    // scheduling barrier keeps that order), so that waiting for K and Q does
    // not wait for these too
    __builtin_amdgcn_sched_barrier(0);
    const int jbase = jbeg - jbeg % NH;
    load_gb(jbase);
    if constexpr (CONV) {
#pragma unroll
        for (int j = 0; j < NHK; ++j)
            if (tid + NT * j < 6 * DK) sA[tid + NT * j] = hk[j];
        // sA: the history [3][q | k], then the taps [q | k] (float4 each)
        float4 *sW = reinterpret_cast<float4 *>(sA + 6 * DK);
        if (tid < 2 * DK) sW[tid] = wt;
        lds_sync();
        conv_rows<E, KL>(kraw, sW + DK + kcv * VEC, krow0, len, sA, 2 * DK, DK + kcv * VEC, kx, SI ? kxl : nullptr);
        conv_rows<E, KL>(qraw, sW + kcv * VEC, krow0, len, sA, 2 * DK, kcv * VEC, qx, SI ? qxl : nullptr);
    }
#pragma unroll
    for (int p = 0; p < KL; ++p) {
        const int r = CONV ? krow0 + p : (tid + NT * p) / VPR;
        const int cv = kcv;
        const u32x4 kv = r < len ? kx[p] : u32x4{0u, 0u, 0u, 0u};
        const u32x4 qv = r < len ? qx[p] : u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4 *>(sK + r * LDK + cv * VEC) = kv;
        *reinterpret_cast<u32x4 *>(sX + r * LDX + cv * VEC) = qv;
        float k2, q2;
        if constexpr (SI) {
            // norms of the two-term rows (hi + lo), already zero past the end
            *reinterpret_cast<u32x4 *>(sKL + r * LDK + cv * VEC) = kxl[p];
            *reinterpret_cast<u32x4 *>(sXL + r * LDX + cv * VEC) = qxl[p];
            float a[VEC], b[VEC], c[VEC], d[VEC];
            unpack16<E>(kv, a);
            unpack16<E>(kxl[p], b);
            unpack16<E>(qv, c);
            unpack16<E>(qxl[p], d);
            k2 = 0.f;
            q2 = 0.f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                k2 += (a[e] + b[e]) * (a[e] + b[e]);
                q2 += (c[e] + d[e]) * (c[e] + d[e]);
            }
        } else {
            k2 = sumsq16<E>(kv);
            q2 = sumsq16<E>(qv);
        }
        // a row's VPR vectors sit in VPR consecutive lanes
        k2 = group_sum<VPR>(k2);
        q2 = group_sum<VPR>(q2);
        if (cv == 0) {
            sRK[r] = r < len ? rsqrtf(k2 + pp.eps) : 0.f;
            sRQ[r] = r < len ? rsqrtf(q2 + pp.eps) * pp.scale : 0.f;
        }
    }
    lds_sync();
    head_scalars(jbase);
    // The first value head's V rows, issued only now: every workgroup of a
    // round starts by loading its rows at once, and K and Q (which the norms
    // wait for) arrive sooner without V competing for the same bandwidth; V
    // is first used after the fragment stores and the K K^T products.
    load_v(kh * ratio + jbeg, true);

    // 2. raw q and k^T of this key head as operand fragments for the scan
    {
        char *kb_blk = pp.kblocks + ((size_t)slot * pp.H_k + kh) * ((size_t)G::KBLK * 1024);
        static_assert(G::NQF % NW == 0 && G::NKF % NW == 0, "fragments per wave");
#pragma unroll
        for (int ff = 0; ff < G::NQF / NW; ++ff) {
            const int f = w + NW * ff;
            const int rt = f / NKD, kb = f % NKD;
            store_frag<E>(kb_blk + G::F_Q * 1024, f, lane, M::load_rm(sX + (16 * rt + n) * LDX, kb * KB, qd));
            if constexpr (SI)
                store_frag<E>(kb_blk + G::F_QL * 1024, f, lane, M::load_rm(sXL + (16 * rt + n) * LDX, kb * KB, qd));
        }
#pragma unroll
        for (int ff = 0; ff < G::NKF / NW; ++ff) {
            const int f = w + NW * ff;
            const int mt = f / NKC, kc = f % NKC;
            store_frag<E>(kb_blk + G::F_KT * 1024, f, lane, TR::frag(sK, LDK, kc * KB, 16 * mt, lane));
            if constexpr (SI)
                store_frag<E>(kb_blk + G::F_KTL * 1024, f, lane, TR::frag(sKL, LDK, kc * KB, 16 * mt, lane));
        }
    }

    // 3. raw K K^T (lower tiles) and K Q^T (tiles (ct, rt), ct <= rt): 20
    //    tile products, tile it = w + NW s in wave w (5 per wave, or 3 and 2
    //    with eight waves); kept in registers for all value heads.
    constexpr int NPW = (20 + NW - 1) / NW;
    floatx4 acc[NPW];
#pragma unroll
    for (int s = 0; s < NPW; ++s) {
        acc[s] = floatx4{0.f, 0.f, 0.f, 0.f};
        const int it = prod_it<NW>(w, s);
        if (it < 0 || it >= 20) continue;     // wave-uniform; LDS reads and matrix-core ops only
        const int pr = it < 10 ? it : it - 10;
        const int rt = low_r(pr), ct = low_c(pr);
        const int ka = (16 * (it < 10 ? rt : ct) + n) * LDK;
        const int kbo = it < 10 ? (16 * ct + n) * LDK : (16 * rt + n) * LDX;
        const E *ra = sK + ka;
        const E *rb = (it < 10 ? sK : sX) + kbo;
#pragma unroll
        for (int kb = 0; kb < NKD; ++kb) {
            const Frag fa = M::load_rm(ra, kb * KB, qd), fb = M::load_rm(rb, kb * KB, qd);
            M::mma(acc[s], fa, fb);
            if constexpr (SI) {
                // (a_h + a_l)(b_h + b_l) without the lo x lo term
                M::mma(acc[s], M::load_rm(sKL + ka, kb * KB, qd), fb);
                M::mma(acc[s], fa, M::load_rm((it < 10 ? sKL : sXL) + kbo, kb * KB, qd));
            }
        }
    }
    lds_sync();   // Q is dead: sX holds V from here on

    for (int jv = jbeg; jv < jend; ++jv) {
        // With eight waves the lane index is made opaque once per head, so
        // that the per-lane LDS offsets and store addresses of the head's
        // phases are formed inside the loop: hoisted out of it, they held
        // about 60 registers across all heads, more than four waves per SIMD
        // leave.
        int tid_o = threadIdx.x;
        if constexpr (NW == 8) asm volatile("" : "+v"(tid_o));
        const int tid = tid_o, lane = tid & 63, n = lane & 15, qd = lane >> 4;
        const int h = kh * ratio + jv;
        char *blk = pp.vblocks + ((size_t)slot * pp.H_v + h) * ((size_t)G::VBLK * 1024);
        char *Wf = blk + G::F_W * 1024;
        char *Wlf = blk + G::F_WL * 1024;
        char *Pf = blk + G::F_PH * 1024;
        char *Plf = blk + G::F_PL * 1024;
        char *U0f = blk + G::F_U0 * 1024;
        const int hs = jv % NH;
        const double *sG = sGh + hs * C;
        const float *sRA = sRAh + hs * C, *sBeta = sBetah + hs * C, *sCol = sColh + hs * C;

        // 4a. V rows of this head; row scalars of the next NH heads
        if constexpr (!CONV) {
#pragma unroll
            for (int p = 0; p < VL; ++p) {
                const int vi = tid + NT * p;
                if (vi < C * VPRV)
                    *reinterpret_cast<u32x4 *>(sX + (vi / VPRV) * LDX + (vi % VPRV) * VEC) = vpre[p];
            }
        } else {
            // raw rows into sX and the head's history rows [m][DV] into sA
            // (free here); then each thread takes its rows and the three
            // before them, and after a second barrier writes the prologue's
            // result over the raw rows
            u32x4 xv[VL + 3];
#pragma unroll
            for (int p = 0; p < VL; ++p) {
                xv[p + 3] = vpre[p];
                *reinterpret_cast<u32x4 *>(sX + (vrow0 + p) * LDX + vcv * VEC) = vpre[p];
            }
#pragma unroll
            for (int j = 0; j < NHV; ++j)
                if (tid + NT * j < 3 * DV) sA[tid + NT * j] = vh[j];
#pragma unroll
            for (int j = 0; j < NWV; ++j)
                if (tid + NT * j < 4 * DV) sA[3 * DV + tid + NT * j] = vw[j];
            lds_sync();
#pragma unroll
            for (int u = 0; u < 3; ++u)
                xv[u] = *reinterpret_cast<const u32x4 *>(sX + max(vrow0 - 3 + u, 0) * LDX + vcv * VEC);
            u32x4 res[VL], resl[SI ? VL : 1];
            conv_rows<E, VL>(xv, reinterpret_cast<const float4 *>(sA + 3 * DV) + vcv * VEC, vrow0, len, sA, DV,
                             vcv * VEC, res, SI ? resl : nullptr);
            lds_sync();
#pragma unroll
            for (int p = 0; p < VL; ++p) {
                *reinterpret_cast<u32x4 *>(sX + (vrow0 + p) * LDX + vcv * VEC) = res[p];
                if constexpr (SI) *reinterpret_cast<u32x4 *>(sXL + (vrow0 + p) * LDX + vcv * VEC) = resl[p];
            }
        }
        load_v(kh * ratio + min(jv + 1, jend - 1), jv + 1 < jend);    // next head (none after the last)
        if (jv > jbase && hs == 0) {
            load_gb(jv);
            head_scalars(jv);
        }
        lds_sync();

        // 4b. A (strictly lower) -> LDS; masked, decayed Q.K -> P fragments.
        //     exp is always taken of G_r - G_c <= 0 (fp64 difference).
        auto a_tile = [&](int s) {
                // lane: column c, rows r0 + j
                const int it = prod_it<NW>(w, s);
                const int rt = low_r(it), ct = low_c(it);
                const int c = 16 * ct + n, r0 = 16 * rt + 4 * qd;
                const double gc = sG[c];
                const float fc = sRK[c];
                const double2 g01 = *reinterpret_cast<const double2 *>(sG + r0);
                const double2 g23 = *reinterpret_cast<const double2 *>(sG + r0 + 2);
                const floatx4 fr = *reinterpret_cast<const floatx4 *>(sRA + r0);
                const double gr[4] = {g01.x, g01.y, g23.x, g23.y};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float e = exp_neg(gr[j] - gc);
                    sA[(r0 + j) * LDA + c] = (c < r0 + j) ? fr[j] * fc * acc[s][j] * e : 0.f;
                }
        };
        auto p_val = [&](int s) -> floatx4 {
                // lane: row r, columns c0 + j
                const int pr = prod_it<NW>(w, s) - 10;
                const int rt = low_r(pr), ct = low_c(pr);
                const int r = 16 * rt + n, c0 = 16 * ct + 4 * qd;
                const double gr = sG[r];
                const float fr = sRQ[r];
                const double2 g01 = *reinterpret_cast<const double2 *>(sG + c0);
                const double2 g23 = *reinterpret_cast<const double2 *>(sG + c0 + 2);
                const floatx4 fc = *reinterpret_cast<const floatx4 *>(sRK + c0);
                const double gc[4] = {g01.x, g01.y, g23.x, g23.y};
                floatx4 pv;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float e = exp_neg(gr - gc[j]);
                    pv[j] = (c0 + j <= r) ? fr * fc[j] * acc[s][j] * e : 0.f;
                }
                return pv;
        };
        auto p_tile = [&](int s) {
                const int pr = prod_it<NW>(w, s) - 10;
                const int rt = low_r(pr), ct = low_c(pr);
                store_quarter2<E>(Pf, Plf, rt * NKC + ct / TPB, lane, ct % TPB, p_val(s));
        };
        // tiles 0..9 are A tiles, 10..19 P tiles (see prod_it).  Four waves:
        // w and w + 4 are A tiles for every wave, w + 12 and w + 16 P tiles,
        // w + 8 an A tile for waves 0, 1 and a P tile for 2, 3.  Eight waves:
        // each wave's P tiles fill whole fragments, written at once.
        if constexpr (NW == 4) {
            a_tile(0);
            a_tile(1);
            p_tile(3);
            p_tile(4);
            if (w < 2) a_tile(2); else p_tile(2);
        } else {
            a_tile(0);
            if (w < 2) {
                a_tile(1);
                if constexpr (TPB == 2) {
                    const int pr = prod_it<NW>(w, 2) - 10;
                    store_pair2(Pf, Plf, low_r(pr) * NKC + low_c(pr) / TPB, lane, p_val(2), floatx4{0.f, 0.f, 0.f, 0.f});
                } else {
                    p_tile(2);
                }
            } else if (w < 6) {
                if constexpr (TPB == 2) {
                    const int pr = prod_it<NW>(w, 1) - 10;
                    store_pair2(Pf, Plf, low_r(pr) * NKC + low_c(pr) / TPB, lane, p_val(1), p_val(2));
                } else {
                    p_tile(1);
                    p_tile(2);
                }
            }
        }
        for (int z = w; z < 6; z += NW) {
            const int rt = up_r(z), ct = up_c(z);
            // a fragment wholly above the diagonal is never read by the scan;
            // with eight waves the partly zero ones are written whole above
            if (NW == 4 && (ct / TPB) * KB <= 16 * rt + 15)
                store_quarter2<E>(Pf, Plf, rt * NKC + ct / TPB, lane, ct % TPB, floatx4{0.f, 0.f, 0.f, 0.f});
            // the products with T read whole K blocks: its upper blocks are zero
            *reinterpret_cast<floatx4 *>(sT + (16 * rt + (lane >> 2)) * LDA + 16 * ct + 4 * (lane & 3)) =
                floatx4{0.f, 0.f, 0.f, 0.f};
        }
        lds_sync();

        // 4c. T = (I + A)^-1: diagonal 16x16 blocks by forward substitution
        //     (wave 0, one lane per column of one block)
        if (w == 0) {
            const int b = lane >> 4, j = lane & 15;
            const float *Ab = sA + (16 * b) * LDA + 16 * b;
            // row i of the block is read two rows ahead of its use, so the
            // dependent chain never waits for LDS (the scheduling barriers
            // keep the compiler from hoisting every read to the top)
            floatx4 win[3][4];
            auto rd = [&](int i) {
#pragma unroll
                for (int c4 = 0; c4 < i; c4 += 4) win[i % 3][c4 / 4] = *reinterpret_cast<const floatx4 *>(Ab + i * LDA + c4);
            };
            rd(1);
            float t[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (i + 2 < 16) rd(i + 2);
                float a = (i == j) ? 1.f : 0.f;
#pragma unroll
                for (int c4 = 0; c4 < i; c4 += 4)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (c4 + e < i) a -= win[i % 3][c4 / 4][e] * t[c4 + e];
                t[i] = a;
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sT[(16 * b + i) * LDA + 16 * b + j] = t[i];
        }
        lds_sync();
        //     off-diagonal blocks by distance: T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj
        for (int d = 1; d < 4; ++d) {
            if (w < 4 - d) {
                const int bi = w + d, bj = w;
                floatx4 X = {0.f, 0.f, 0.f, 0.f};
                for (int m = bj; m < bi; ++m) {
                    const floatx4 a = *reinterpret_cast<const floatx4 *>(sA + (16 * bi + n) * LDA + 16 * m + 4 * qd);
                    floatx4 bt;
#pragma unroll
                    for (int j = 0; j < 4; ++j) bt[j] = sT[(16 * m + 4 * qd + j) * LDA + 16 * bj + n];
                    mma_f32_k16(X, a, bt);
                }
                const floatx4 a = -*reinterpret_cast<const floatx4 *>(sT + (16 * bi + n) * LDA + 16 * bi + 4 * qd);
                floatx4 Y = {0.f, 0.f, 0.f, 0.f};
                mma_f32_k16(Y, a, X);
#pragma unroll
                for (int j = 0; j < 4; ++j) sT[(16 * bi + 4 * qd + j) * LDA + 16 * bj + n] = Y[j];
            }
            lds_sync();
        }

        // 4d. W^T = K^T T''^T, T'' = T diag(beta e^G / |k|): wave w takes token
        //     tile tt = w mod 4 (B operand loaded once) and its share of the
        //     dk tiles (all of them with four waves, half with eight).
        //     U0 = T diag(beta) V: wave w takes token tile 3 - w mod 4 and its
        //     share of the column tiles, so every wave runs the same number of
        //     products.
        constexpr int NSH = NW / 4;
        const int sh = w / 4;
        static_assert(NMT % NSH == 0 && NCT % NSH == 0, "tiles per share");
        {
            const int tt = w % 4;
            const int nkb = (16 * tt + 15) / KB + 1;    // K blocks reaching the diagonal
            Frag bh[NKC], bl[NKC];
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb)
                if (kb < nkb) SP::rm_f32(sT + (16 * tt + n) * LDA, kb * KB, qd, sCol, bh[kb], bl[kb]);
            floatx4 wprev = {0.f, 0.f, 0.f, 0.f};   // bf16: the first half of a fragment
#pragma unroll
            for (int dd = 0; dd < NMT / NSH; ++dd) {
                const int dt = sh * (NMT / NSH) + dd;
                floatx4 a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb) {
                    if (kb >= nkb) break;
                    const Frag a = TR::frag(sK, LDK, kb * KB, 16 * dt, lane);
                    M::mma(a4, a, bh[kb]);
                    if constexpr (NS == 2) M::mma(a4, a, bl[kb]);
                    if constexpr (SI) M::mma(a4, TR::frag(sKL, LDK, kb * KB, 16 * dt, lane), bh[kb]);
                }
                if constexpr (TPB == 2) {
                    // both halves of the fragment in one store
                    if (dd % 2 == 0) {
                        wprev = a4;
                    } else {
                        if constexpr (SI) store_pair2(Wf, Wlf, tt * NKD + dt / TPB, lane, wprev, a4);
                        else store_pair(Wf, tt * NKD + dt / TPB, lane, wprev, a4);
                    }
                } else {
                    if constexpr (SI) store_quarter2<E>(Wf, Wlf, tt * NKD + dt / TPB, lane, dt % TPB, a4);
                    else store_quarter<E>(Wf, tt * NKD + dt / TPB, lane, dt % TPB, a4);
                }

            }
        }
        {
            const int rt = 3 - w % 4;
            const int nkb = (16 * rt + 15) / KB + 1;
            Frag ah[NKC], al[NKC];
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb)
                if (kb < nkb) SP::rm_f32(sT + (16 * rt + n) * LDA, kb * KB, qd, sBeta, ah[kb], al[kb]);
#pragma unroll
            for (int cc = 0; cc < NCT / NSH; ++cc) {
                const int ct = sh * (NCT / NSH) + cc;
                floatx4 a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb) {
                    if (kb >= nkb) break;
                    const Frag b = TR::frag(sX, LDX, kb * KB, 16 * ct, lane);
                    M::mma(a4, ah[kb], b);
                    if constexpr (NS == 2) M::mma(a4, al[kb], b);
                    if constexpr (SI) M::mma(a4, ah[kb], TR::frag(sXL, LDX, kb * KB, 16 * ct, lane));
                }
                *(reinterpret_cast<floatx4 *>(U0f) + (size_t)(ct * 4 + rt) * 64 + lane) = a4;
            }
        }
        lds_sync();
    }
    // Debug record of the requested chunk and head (launched with one value
    // head per workgroup, so that the head's G, T, column scalars and K are
    // still in LDS here and nothing else is live): G, T, and W from the
    // products of 4d again (same operands, same order).
    if (pp.dbg && jend - jbeg == 1 && kh * ratio + jbeg == pp.dbg_h && pp.dbg_t >= t0 && pp.dbg_t < t0 + len) {
        const int hs = jbeg % NH;
        const double *sG = sGh + hs * C;
        const float *sCol = sColh + hs * C;
        for (int x = tid; x < C * C; x += NT) pp.dbg->T[x / C][x % C] = sT[(x / C) * LDA + x % C];
        if (tid < C) pp.dbg->G[tid] = sG[tid];
        if (tid == 0) {
            pp.dbg->chunk = chunk;
            pp.dbg->t0 = t0;
            pp.dbg->len = len;
            pp.dbg->prepared = 1;
        }
        const int tt = w;
        const int nkb = (16 * tt + 15) / KB + 1;
#pragma unroll 1
        for (int dt = 0; dt < (tt < 4 ? NMT : 0); ++dt) {     // token tiles 0..3: waves 0..3
            floatx4 a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
            for (int kb = 0; kb < nkb; ++kb) {
                Frag bh, bl;
                SP::rm_f32(sT + (16 * tt + n) * LDA, kb * KB, qd, sCol, bh, bl);
                const Frag a = TR::frag(sK, LDK, kb * KB, 16 * dt, lane);
                M::mma(a4, a, bh);
                if constexpr (NS == 2) M::mma(a4, a, bl);
                if constexpr (SI) M::mma(a4, TR::frag(sKL, LDK, kb * KB, 16 * dt, lane), bh);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) pp.dbg->W[16 * tt + n][16 * dt + 4 * qd + j] = a4[j];
        }
    }
}

// --------------------------------------------------------------------------
// 3. sequential state scan + output
// --------------------------------------------------------------------------
struct ScanParams {
    const float *state_in;
    float *state_out;
    void *out;
    const int32_t *slot_in, *slot_out;
    const int32_t *cstart;
    const ChunkEntry *ent;
    const char *vblocks, *kblocks;
    int H_k, H_v;
    int64_t slot_stride;
    int single_T;      // >= 0: one sequence of this many tokens, no chunk table
    // chunks [seg_lo, seg_hi) of the batch, the seg_idx-th range; a sequence
    // that began in an earlier range takes its state from the carry state of
    // the previous range's parity, one that goes on past this range leaves
    // it in the carry state of this range's parity ([2][H_v][DK][DV] fp32).
    // At most one sequence crosses each range boundary, and consecutive
    // ranges use the two states in turn, so the reads of one launch never
    // meet its writes.
    int seg_lo, seg_hi, seg_idx;
    float *carry;
    // debug record (null: off): U of the chunk the preparation recorded, for
    // value head dbg_h
    gdn_debug_chunk *dbg = nullptr;
    int dbg_h = -1;
    // layer prologue (conv_out non-null): the new convolution state of each
    // sequence, the last kConv - 1 inputs of (its state ++ its rows), per
    // channel of the mixed rows conv_x ([T][conv_dim], element type E); the
    // state rows of slot s start at conv_in / conv_out + s * slot_stride
    const void *conv_x = nullptr;
    const float *conv_in = nullptr;
    float *conv_out = nullptr;
    int conv_dim = 0;
};

template <int DK, int DV, int CT, typename E> struct ScanLds {
    using G = Geo<DK, DV, E>;      // (the q/k split does not change the exchange)
    // exchange only, per column tile: the state as two-term B fragments per
    // dk block, and the chunk deltas U and ks*U as two-term B fragments per
    // token block (each 1 KiB = 64 lanes x 16 bytes)
    static constexpr int NSP = Split<E>::N;
    static constexpr size_t SF = (size_t)CT * G::NKD * NSP * 1024;
    static constexpr size_t UF = (size_t)CT * G::NKC * NSP * 1024;
    static constexpr size_t BYTES = SF + 2 * UF;
};

// The four row scalars of a lane's accumulator rows (4 qd + j, j = 0..3)
// from one value per lane (lane 4 m + j of each quad holds row j's): DPP
// quad broadcasts, so a wave's load returns 4 instead of 16 bytes per lane
// through the CU's data-return path, which the scan keeps busy.
__device__ __forceinline__ floatx4 quad_rows(float x)
{
    const int b = __float_as_int(x);
    return floatx4{__int_as_float(__builtin_amdgcn_mov_dpp(b, 0x00, 0xf, 0xf, true)),
                   __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x55, 0xf, 0xf, true)),
                   __int_as_float(__builtin_amdgcn_mov_dpp(b, 0xAA, 0xf, 0xf, true)),
                   __int_as_float(__builtin_amdgcn_mov_dpp(b, 0xFF, 0xf, 0xf, true))};
}

// Two-term conversion of one accumulator tile (4 values per lane).  For bf16
// operands it fills `part` (0 or 1) of a K block's 16-byte lane slot: 8 bytes
// of hi and 8 bytes of lo bf16; fp32 operands have a single term filling the
// whole slot.
template <typename E> struct TileOut;
template <> struct TileOut<bf16_t> {
    __device__ static __forceinline__ void put(u32x4 *hi, u32x4 *lo, int lane, int part, floatx4 v) {
        bf16x4 h, l;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            h[j] = (__bf16)v[j];
            l[j] = (__bf16)(v[j] - (float)h[j]);
        }
        *reinterpret_cast<bf16x4 *>(reinterpret_cast<char *>(hi + lane) + 8 * part) = h;
        *reinterpret_cast<bf16x4 *>(reinterpret_cast<char *>(lo + lane) + 8 * part) = l;
    }
};
template <> struct TileOut<float> {
    __device__ static __forceinline__ void put(u32x4 *hi, u32x4 *lo, int lane, int part, floatx4 v) {
        (void)lo;
        (void)part;
        hi[lane] = __builtin_bit_cast(u32x4, v);
    }
};

// Scan over a sequence's chunks for one value head and CT column tiles of 16
// state columns, with two sets of four waves per column tile:
//   state waves (role 0), wave rt: U = U0 - W S for token rows 16*rt.. in
//     phase A (published with ks*U for the update); in phase B the update of
//     the owned dk blocks kb = rt (mod 4) of the state, S = gn S + K^T (ks U).
//   output waves (role 1), wave rt: the inter-chunk read-out Q S for token
//     rows 16*rt.. in phase A, then O = qs (Q S) + P U and its store.
// Each set's chain per chunk is half of a single wave's, and every SIMD holds
// one wave of each set.  Every operand of a chunk is loaded from the
// workspace straight into the registers of the wave that uses it, re-issued
// for the next chunk right after its last use in this one, so its latency
// overlaps a chunk of work; LDS carries only the per-chunk exchange (state
// and delta fragments).
template <int DK, int DV, int CT, typename E, typename OT, bool SI>
__global__ __launch_bounds__(CT * 512) void scan_kernel(ScanParams sp)
{
    using M = Mfma<E>;
    using SP = Split<E>;
    using G = Geo<DK, DV, E, SI>;
    using L = ScanLds<DK, DV, CT, E>;
    using Frag = typename M::Frag;
    constexpr int KB = M::KB, TPB = M::TPB, NS = SP::N;
    constexpr int NKD = G::NKD, NKC = G::NKC;
    constexpr int NOWN = (NKD + 3) / 4;           // dk blocks of the state owned per wave (max)

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    u32x4 *sSf = reinterpret_cast<u32x4 *>(smem);                         // [CT][NKD][NS][64]
    u32x4 *sUf = reinterpret_cast<u32x4 *>(smem + L::SF);                 // [CT][NKC][NS][64]
    u32x4 *sKf = reinterpret_cast<u32x4 *>(smem + L::SF + L::UF);         // [CT][NKC][NS][64]

    // grid (value head, column tile, sequence): the column tiles of a head sit
    // H_v workgroups apart, so with H_v a multiple of 8 they share an XCD
    // (and its L2, which serves their common operand fragments)
    // Workgroups go to the eight XCDs in turn by linear block index, so
    // blockIdx.x % 8 is this workgroup's XCD whenever H_v % 8 == 0.  Giving
    // each XCD a contiguous run of value heads puts the heads of one key head
    // on one XCD, whose L2 then fetches the key head's q and k^T fragments
    // once (at T=4096 with Qwen3-Next heads the scan's fetched bytes drop
    // from 205 to 171 MB per launch).
    const int h = sp.H_v % 8 == 0 ? (blockIdx.x % 8) * (sp.H_v / 8) + blockIdx.x / 8 : blockIdx.x;
    const int cg = blockIdx.y, i = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int ctl = wv >> 3, role = (wv >> 2) & 1, rt = wv & 3;
    const int n = lane & 15, qd = lane >> 4;
    const int kh = h / (sp.H_v / sp.H_k);
    const int ct = cg * CT + ctl;
    const int col0 = 16 * ct;

    auto xfrag = [&](const u32x4 *base, int f) -> Frag { return __builtin_bit_cast(Frag, base[f * 64 + lane]); };
    u32x4 *mySf = sSf + ctl * (NKD * NS * 64);
    u32x4 *myUf = sUf + ctl * (NKC * NS * 64);
    u32x4 *myKf = sKf + ctl * (NKC * NS * 64);

    const bool single = sp.single_T >= 0;
    const int cs_seq = single ? 0 : sp.cstart[i];
    const int ce_seq = single ? (sp.single_T + C - 1) / C : sp.cstart[i + 1];
    // this launch's part of the sequence; an empty sequence (state copied
    // through) belongs to the first range
    const bool empty = cs_seq >= ce_seq;
    const int cs = empty ? cs_seq : max(cs_seq, sp.seg_lo);
    const int ce = empty ? cs_seq : min(ce_seq, sp.seg_hi);
    if (empty ? sp.seg_lo != 0 : cs >= ce) return;      // uniform over the workgroup
    const bool carried_in = !empty && cs_seq < sp.seg_lo;
    const bool carried_out = !empty && ce_seq > sp.seg_hi;
    const float *carry_in = sp.carry + ((int64_t)((sp.seg_idx + 1) & 1) * sp.H_v + h) * DK * DV + col0 + n;
    float *carry_out = sp.carry + ((int64_t)(sp.seg_idx & 1) * sp.H_v + h) * DK * DV + col0 + n;
    const size_t vstride = (size_t)G::VBLK * 1024, kstride = (size_t)G::KBLK * 1024;
    const char *vbase = sp.vblocks + (size_t)h * vstride;
    const char *kbase = sp.kblocks + (size_t)kh * kstride;
    const size_t vstep = (size_t)sp.H_v * vstride, kstep = (size_t)sp.H_k * kstride;
    // chunk c of this range has its factors in slot c - seg_lo (c >= seg_lo
    // for every chunk read: an empty sequence reads chunk 0 and only in the
    // range that starts at 0)
    auto vblk = [&](int c) { return reinterpret_cast<const u32x4 *>(vbase + (size_t)(c - sp.seg_lo) * vstep); };
    auto kblk = [&](int c) { return reinterpret_cast<const u32x4 *>(kbase + (size_t)(c - sp.seg_lo) * kstep); };
    auto vfrag = [&](int c, int f) -> Frag { return __builtin_bit_cast(Frag, vblk(c)[f * 64 + lane]); };
    auto kfrag = [&](int c, int f) -> Frag { return __builtin_bit_cast(Frag, kblk(c)[f * 64 + lane]); };
    auto scal1 = [&](int c, int off) -> float {
        return reinterpret_cast<const float *>(vblk(c) + G::F_SCAL * 64)[off];
    };
    const int ro = 16 * rt + 4 * qd;               // first of this lane's 4 token rows
    // operands of the first chunk (a sequence without chunks reads chunk 0
    // and runs no iteration)
    const int c0 = cs < ce ? cs : 0;

    if (role == 0) {
        // state: registers of the owning wave, published as two-term B fragments
        // (loaded first, published once the first chunk's operands are in
        // flight too, so that the two latencies overlap)
        floatx4 Sreg[NOWN][TPB];
        {
            const int sin = sp.state_in ? sp.slot_in[i] : -1;
            const float *base = carried_in ? carry_in
                              : sin >= 0   ? sp.state_in + (int64_t)sin * sp.slot_stride + (int64_t)h * DK * DV + col0 + n
                                           : nullptr;
#pragma unroll
            for (int o = 0; o < NOWN; ++o) {
                const int kb = rt + 4 * o;
#pragma unroll
                for (int t = 0; t < TPB; ++t) {
                    floatx4 v = {0.f, 0.f, 0.f, 0.f};
                    if (base && kb < NKD) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) v[j] = base[(int64_t)(16 * (kb * TPB + t) + 4 * qd + j) * DV];
                    }
                    Sreg[o][t] = v;
                }
            }
        }
        const int u0f = G::F_U0 + ct * 4 + rt;     // accumulator tile (ct, rt) of U0
        Frag Wf[NKD], Wlf[SI ? NKD : 1], Kf[NOWN * TPB][NKC], Klf[SI ? NOWN * TPB : 1][NKC];
#pragma unroll
        for (int kb = 0; kb < NKD; ++kb) {
            Wf[kb] = vfrag(c0, G::F_W + rt * NKD + kb);
            if constexpr (SI) Wlf[kb] = vfrag(c0, G::F_WL + rt * NKD + kb);
        }
#pragma unroll
        for (int o = 0; o < NOWN; ++o)
#pragma unroll
            for (int t = 0; t < TPB; ++t) {
                const int mt = min(rt + 4 * o, NKD - 1) * TPB + t;
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc) {
                    Kf[o * TPB + t][kc] = kfrag(c0, G::F_KT + mt * NKC + kc);
                    if constexpr (SI) Klf[o * TPB + t][kc] = kfrag(c0, G::F_KTL + mt * NKC + kc);
                }
            }
        floatx4 u0 = __builtin_bit_cast(floatx4, vblk(c0)[u0f * 64 + lane]);
        float ks1 = scal1(c0, 64 + ro + (n & 3));
        float gn = scal1(c0, 128);
        // debug record: the chunk whose U is recorded (-1: none here)
        int dbg_c = -1;
        if (sp.dbg && h == sp.dbg_h) dbg_c = __builtin_amdgcn_readfirstlane(sp.dbg->chunk);
        // Let the state and the first chunk's operands land before the loop:
        // the loop's waits then only have to account for the loads issued
        // inside it.
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
#pragma unroll
        for (int o = 0; o < NOWN; ++o) {
            const int kb = rt + 4 * o;
#pragma unroll
            for (int t = 0; t < TPB; ++t)
                if (kb < NKD) TileOut<E>::put(mySf + (kb * NS) * 64, mySf + (kb * NS + NS - 1) * 64, lane, t, Sreg[o][t]);
        }
        lds_sync();

        for (int c = cs; c < ce; ++c) {
            const int cn = min(c + 1, ce - 1);     // next chunk (the last one reloads itself)

            // phase A: U = U0 - W S, state from LDS
            floatx4 WSh = {0.f, 0.f, 0.f, 0.f}, WSl = WSh;
#pragma unroll
            for (int kb = 0; kb < NKD; ++kb) {
                const Frag sh = xfrag(mySf, kb * NS);
                M::mma(WSh, Wf[kb], sh);
                if constexpr (NS == 2) M::mma(WSl, Wf[kb], xfrag(mySf, kb * NS + 1));
                Wf[kb] = vfrag(cn, G::F_W + rt * NKD + kb);
                if constexpr (SI) {
                    M::mma(WSl, Wlf[kb], sh);
                    Wlf[kb] = vfrag(cn, G::F_WL + rt * NKD + kb);
                }
            }
            const floatx4 U = u0 - (WSh + WSl);
            const floatx4 Uk = U * quad_rows(ks1);
            if (c == dbg_c) {
                const __amdgpu_buffer_rsrc_t dbg_u = raw_buffer(&sp.dbg->U[0][0], (uint32_t)sizeof(sp.dbg->U));
#pragma unroll
                for (int j = 0; j < 4; ++j) buffer_store(U[j], dbg_u, (uint32_t)(((ro + j) * 128 + col0 + n) * 4));
                if (ct == 0 && rt == 0 && lane == 0) sp.dbg->scanned = 1;
            }
            u0 = __builtin_bit_cast(floatx4, vblk(cn)[u0f * 64 + lane]);
            ks1 = scal1(cn, 64 + ro + (n & 3));
            {
                const int kc = rt / TPB, part = rt % TPB;
                TileOut<E>::put(myUf + (kc * NS) * 64, myUf + (kc * NS + NS - 1) * 64, lane, part, U);
                TileOut<E>::put(myKf + (kc * NS) * 64, myKf + (kc * NS + NS - 1) * 64, lane, part, Uk);
            }
            // region order: matrix-core op, load, alternately
#pragma unroll
            for (int q = 0; q < NKD; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, NS, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                if constexpr (SI) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
            }
            lds_sync();

            // phase B: the owned blocks of the state
            if (rt < NKD) {
                Frag kh_[NKC], kl_[NKC];
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc) {
                    kh_[kc] = xfrag(myKf, kc * NS);
                    kl_[kc] = xfrag(myKf, kc * NS + NS - 1);
                }
#pragma unroll
                for (int o = 0; o < NOWN; ++o) {
                    const int kb = rt + 4 * o;
                    if (kb >= NKD) continue;
                    floatx4 Sa[TPB], Sb[TPB];
#pragma unroll
                    for (int t = 0; t < TPB; ++t) {
                        Sa[t] = Sreg[o][t] * gn;
                        Sb[t] = floatx4{0.f, 0.f, 0.f, 0.f};
                    }
#pragma unroll
                    for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                        for (int t = 0; t < TPB; ++t) {
                            M::mma(Sa[t], Kf[o * TPB + t][kc], kh_[kc]);
                            if constexpr (NS == 2) M::mma(Sb[t], Kf[o * TPB + t][kc], kl_[kc]);
                            Kf[o * TPB + t][kc] = kfrag(cn, G::F_KT + ((rt + 4 * o) * TPB + t) * NKC + kc);
                            if constexpr (SI) {
                                M::mma(Sb[t], Klf[o * TPB + t][kc], kh_[kc]);
                                Klf[o * TPB + t][kc] = kfrag(cn, G::F_KTL + ((rt + 4 * o) * TPB + t) * NKC + kc);
                            }
                        }
#pragma unroll
                    for (int t = 0; t < TPB; ++t) {
                        Sreg[o][t] = Sa[t] + Sb[t];
                        TileOut<E>::put(mySf + (kb * NS) * 64, mySf + (kb * NS + NS - 1) * 64, lane, t, Sreg[o][t]);
                    }
                }
            }
            gn = scal1(cn, 128);
            // region order: matrix-core op, load, alternately
#pragma unroll
            for (int q = 0; q < NOWN * TPB * NKC; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, NS, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                if constexpr (SI) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
            }
            lds_sync();
        }

        const int sout = sp.slot_out[i];
        if (carried_out || sout >= 0) {
            float *base = carried_out ? carry_out : sp.state_out + (int64_t)sout * sp.slot_stride + (int64_t)h * DK * DV + col0 + n;
#pragma unroll
            for (int o = 0; o < NOWN; ++o) {
                const int kb = rt + 4 * o;
                if (kb >= NKD) continue;
#pragma unroll
                for (int t = 0; t < TPB; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        base[(int64_t)(16 * (kb * TPB + t) + 4 * qd + j) * DV] = Sreg[o][t][j];
            }
        }
    } else {
        OT *og = static_cast<OT *>(sp.out);
        Frag Qf[NKD], Qlf[SI ? NKD : 1], Ph[NKC], Pl[NKC];
        // P row tile rt is zero past column 16 rt + 15, so its K blocks from
        // npl on are zero and the preparation does not write them, and phase
        // B skips them.  The one-term kernel reads them through a range that
        // ends before them (zero, no memory access): skipping those loads on
        // the wave-uniform branch made that kernel slower (by about 7%, also
        // with the skipped loads issued first).  The two-term kernel, with
        // twice the fragments per block, skips them.
        const int npl = (16 * rt + 15) / KB + 1;
        auto pfrag = [&](int c, int base, int kc) -> Frag {
            const auto r = raw_buffer(const_cast<u32x4 *>(vblk(c)) + (size_t)(base + rt * NKC) * 64, (uint32_t)npl * 1024u);
            return __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)(kc * 64 + lane) * 16u, 0, 0));
        };
#pragma unroll
        for (int kb = 0; kb < NKD; ++kb) {
            Qf[kb] = kfrag(c0, G::F_Q + rt * NKD + kb);
            if constexpr (SI) Qlf[kb] = kfrag(c0, G::F_QL + rt * NKD + kb);
        }
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            if (SI && kc >= npl) continue;
            Ph[kc] = pfrag(c0, G::F_PH, kc);
            if constexpr (NS == 2) Pl[kc] = pfrag(c0, G::F_PL, kc);
        }
        float qs1 = scal1(c0, ro + (n & 3));
        // the sequence's token range; its chunks are consecutive 64-token pieces
        const int tbeg = single ? C * cs : cs >= ce ? 0 : sp.ent[cs].t0;
        const int tend = single ? sp.single_T : cs < ce ? sp.ent[ce - 1].t0 + sp.ent[ce - 1].len : 0;
        const uint32_t row_bytes = (uint32_t)(sp.H_v * DV * sizeof(OT));
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
        lds_sync();

        for (int c = cs; c < ce; ++c) {
            const int cn = min(c + 1, ce - 1);

            // phase A: the inter-chunk read-out Q S, state from LDS
            floatx4 OQh = {0.f, 0.f, 0.f, 0.f}, OQl = OQh;
#pragma unroll
            for (int kb = 0; kb < NKD; ++kb) {
                const Frag sh = xfrag(mySf, kb * NS);
                M::mma(OQh, Qf[kb], sh);
                if constexpr (NS == 2) M::mma(OQl, Qf[kb], xfrag(mySf, kb * NS + 1));
                Qf[kb] = kfrag(cn, G::F_Q + rt * NKD + kb);
                if constexpr (SI) {
                    M::mma(OQl, Qlf[kb], sh);
                    Qlf[kb] = kfrag(cn, G::F_QL + rt * NKD + kb);
                }
            }
            const floatx4 Oi = (OQh + OQl) * quad_rows(qs1);
            qs1 = scal1(cn, ro + (n & 3));
#pragma unroll
            for (int q = 0; q < NKD; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, NS, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                if constexpr (SI) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
            }
            lds_sync();

            // phase B: intra-chunk output P U
            floatx4 Oa = Oi, Ob = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                if (kc * KB > 16 * rt + 15) continue;
                const Frag uh = xfrag(myUf, kc * NS);
                M::mma(Oa, Ph[kc], uh);
                if constexpr (NS == 2) {
                    M::mma(Ob, Ph[kc], xfrag(myUf, kc * NS + 1));
                    M::mma(Ob, Pl[kc], uh);
                }
            }
            {
                // rows >= len of a partial chunk fall outside the buffer and are dropped
                const int t0 = tbeg + C * (c - cs), len = min(C, tend - t0);
                const __amdgpu_buffer_rsrc_t ob =
                    raw_buffer(og + ((size_t)t0 * sp.H_v + h) * DV + col0, (uint32_t)len * row_bytes);
                const floatx4 O = Oa + Ob;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    buffer_store(from_f32<OT>(O[j]), ob, (uint32_t)(ro + j) * row_bytes + n * (uint32_t)sizeof(OT));
            }
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                if (SI && kc >= npl) continue;
                Ph[kc] = pfrag(cn, G::F_PH, kc);
                if constexpr (NS == 2) Pl[kc] = pfrag(cn, G::F_PL, kc);
            }
            lds_sync();
        }
    }

    // The layer prologue's new convolution state, written by the launch that
    // holds the sequence's last chunk (an empty sequence's, which only copies
    // the state, by the first range's): every preparation that read the old
    // state ran before this launch.  The workgroups of a sequence split its
    // channels: each its column tile of its value head's v channels, and a
    // share of its key head's q and k channels.  One wave each.
    if (sp.conv_out && (empty ? sp.seg_lo == 0 : !carried_out) && role == 1 && rt == 0 && ctl == 0) {
        constexpr int kH = kConv - 1;
        const int sout = sp.slot_out[i];
        if (sout >= 0) {
            const int sin = sp.conv_in ? sp.slot_in[i] : -1;
            int64_t tb = 0, te = 0;
            if (single) {
                te = sp.single_T;
            } else if (!empty) {
                tb = sp.ent[cs_seq].t0;
                te = sp.ent[ce_seq - 1].t0 + sp.ent[ce_seq - 1].len;
            }
            const int64_t len = te - tb;
            const E *x = static_cast<const E *>(sp.conv_x);
            const int ratio = sp.H_v / sp.H_k, ntile = DV / 16;
            const int parts = ratio * ntile, part = (h % ratio) * ntile + ct;
            const int nqk = (2 * DK + parts - 1 - part) / parts;      // q/k channels part + parts * m
            // one lane per channel: its three new values are read before any is written
            for (int m = lane; m < 16 + nqk; m += 64) {
                int64_t ch;
                if (m < 16) {
                    ch = 2 * (int64_t)sp.H_k * DK + (int64_t)h * DV + col0 + m;
                } else {
                    const int c = part + parts * (m - 16);           // of the key head's q then k channels
                    ch = (c < DK ? (int64_t)kh * DK + c : (int64_t)sp.H_k * DK + (int64_t)kh * DK + (c - DK));
                }
                float nu[kH];
#pragma unroll
                for (int jj = 0; jj < kH; ++jj) {
                    const int64_t el = len + jj;                     // element len + jj of (state ++ rows)
                    nu[jj] = el < kH ? (sin >= 0 ? sp.conv_in[(int64_t)sin * sp.slot_stride + ch * kH + el] : 0.f)
                                     : to_f32(x[(tb + el - kH) * sp.conv_dim + ch]);
                }
#pragma unroll
                for (int jj = 0; jj < kH; ++jj) sp.conv_out[(int64_t)sout * sp.slot_stride + ch * kH + jj] = nu[jj];
            }
        }
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
    char *vblocks, *kblocks;
    float *obuf, *carry;
};

WsPtrs ws_ptrs(const Problem &p, const PrefillArgs &a)
{
    WsPtrs w;
    w.L = ws_layout(p, a.n_seqs, a.total_tokens, a.ws_slots);
    char *ws = static_cast<char *>(a.workspace);
    w.hdr = reinterpret_cast<int32_t *>(ws);
    w.ent = reinterpret_cast<ChunkEntry *>(ws + w.L.entries);
    w.cstart = reinterpret_cast<int32_t *>(ws + w.L.cstart);
    w.vblocks = ws + w.L.vblocks;
    w.kblocks = ws + w.L.kblocks;
    w.obuf = reinterpret_cast<float *>(ws + w.L.obuf);
    w.carry = reinterpret_cast<float *>(ws + w.L.carry);
    return w;
}

// Waves per preparation workgroup.  At d_k = d_v = 128 eight: the per-thread
// row vectors and product tiles halve, so two workgroups of eight waves fit a
// CU (128 registers, LDS unchanged) where two of four did, and every phase
// but the triangular solve splits over twice the waves.  Smaller heads keep
// four (their fragment counts do not split eight ways).
template <int DK, int DV> constexpr int kPrepWaves = DK == 128 && DV == 128 ? 8 : 4;

template <int DK, int DV, typename E>
hipError_t prepare_t(const Problem &p, const PrefillArgs &a, const Segment &sg, hipStream_t st)
{
    const WsPtrs w = ws_ptrs(p, a);
    // one sequence: cu_seqlens is [0, total_tokens] by contract, and both
    // kernels derive the chunks arithmetically (no chunk-table launch)
    const bool single = a.n_seqs == 1;
    hipError_t e = hipSuccess;
    if (!single && sg.first) {
        hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(1024), 0, st, a.cu_seqlens, a.n_seqs,
                           (int)a.total_tokens, w.L.max_chunks, w.hdr, w.ent, w.cstart);
        e = hipGetLastError();
    }
    if (e != hipSuccess || a.total_tokens == 0) return e;
    PrepParams pp{a.q, a.k, a.v, a.g, a.beta, w.hdr, w.ent, w.vblocks, w.kblocks,
                  p.H_k, p.H_v, p.scale, p.eps, single ? (int)a.total_tokens : -1,
                  // without raw gates the parameter loads read g (see gates_of in gdn_decode.hip)
                  p.ssm_a ? Gates{p.ssm_a, p.ssm_dt, 1} : Gates{a.g, a.g, 0},
                  p.rs_qk, p.rs_v, p.conv_w,
                  // without a state pool the history loads read the taps (unused)
                  a.conv_in ? a.conv_in : p.conv_w, a.slot_in, p.slot_stride, a.conv_in != nullptr, 0, sg.lo};
    pp.dbg = p.dbg;
    pp.dbg_t = p.dbg_token;
    pp.dbg_h = p.dbg_head;
    const int all = single ? (int)((a.total_tokens + C - 1) / C) : w.L.max_chunks;
    const int chunks = std::min(all, sg.hi) - sg.lo;
    if (chunks <= 0) return hipSuccess;
    // A grid that leaves most workgroup slots empty (e.g. one 512-token
    // ubatch: 8 chunks x 16 key heads) is bound by one workgroup's latency;
    // splitting it by value head halves that chain for a little more work.
    const int per_cu = (sizeof(E) == 2 && !p.conv_w) ? 2 : 1;
    const int ratio = p.H_v / p.H_k;
    if (ratio > 1 && (int64_t)chunks * p.H_v <= (int64_t)per_cu * cu_count()) pp.head_split = 1;
    if (p.dbg && ratio > 1) pp.head_split = 1;     // the debug record is written after the head loop
    const dim3 grid(chunks, pp.head_split ? p.H_v : p.H_k);
    if (p.conv_w) {
        // bf16 rows: two-term bf16 operands (SI); fp32 rows: fp32 operands
        constexpr size_t lds = PrepLds<DK, DV, E, sizeof(E) == 2>::BYTES;
        e = set_lds(prep_kernel<DK, DV, E, true, kPrepWaves<DK, DV>>, lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((prep_kernel<DK, DV, E, true, kPrepWaves<DK, DV>>), grid, dim3(64 * kPrepWaves<DK, DV>), lds,
                           st, pp);
        return hipGetLastError();
    }
    constexpr size_t lds = PrepLds<DK, DV, E>::BYTES;
    e = set_lds(prep_kernel<DK, DV, E, false, kPrepWaves<DK, DV>>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prep_kernel<DK, DV, E, false, kPrepWaves<DK, DV>>), grid, dim3(64 * kPrepWaves<DK, DV>), lds, st,
                       pp);
    return hipGetLastError();
}

template <int DK, int DV, typename E, typename OT, bool SI>
hipError_t scan_t(const Problem &p, const PrefillArgs &a, const Segment &sg, hipStream_t st)
{
    const WsPtrs w = ws_ptrs(p, a);
    constexpr int CT = 1;    // column tiles per workgroup
    void *o = stage_o(p) ? static_cast<void *>(w.obuf) : a.out;
    ScanParams sp{a.state_in, a.state_out, o, a.slot_in, a.slot_out, w.cstart, w.ent,
                  w.vblocks, w.kblocks, p.H_k, p.H_v, p.slot_stride,
                  a.n_seqs == 1 ? (int)a.total_tokens : -1, sg.lo, sg.hi, sg.idx, w.carry};
    sp.dbg = p.dbg;
    sp.dbg_h = p.dbg_head;
    if (p.conv_w) {
        sp.conv_x = a.q;               // the mixed rows (q is their first channel range)
        sp.conv_in = a.conv_in;
        sp.conv_out = a.conv_out;
        sp.conv_dim = p.conv_dim;
    }
    // With several sequences, one scan workgroup per CU: two workgroups on
    // one CU contend for its vector-memory path and LDS (the varlen batch of
    // 12 221 tokens takes 0.39 instead of 0.30 ms in the scan), so the
    // reservation below (more LDS than half a CU holds) keeps them apart.
    constexpr size_t lds_min = ScanLds<DK, DV, CT, E>::BYTES;
    const size_t lds = a.n_seqs > 1 ? std::max<size_t>(lds_min, 96 * 1024) : lds_min;
    hipError_t e = set_lds(scan_kernel<DK, DV, CT, E, OT, SI>, 96 * 1024);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((scan_kernel<DK, DV, CT, E, OT, SI>), dim3(p.H_v, DV / (16 * CT), a.n_seqs),
                       dim3(CT * 512), lds, st, sp);
    e = hipGetLastError();
    if (e == hipSuccess && p.z && sg.last)
        e = launch_gated_norm(p, static_cast<const float *>(o), a.out, a.total_tokens, st);
    return e;
}

template <int DK, int DV>
hipError_t prepare_dv(const Problem &p, const PrefillArgs &a, const Segment &sg, hipStream_t st)
{
    return op_bf16(p) ? prepare_t<DK, DV, bf16_t>(p, a, sg, st) : prepare_t<DK, DV, float>(p, a, sg, st);
}

template <int DK>
hipError_t prepare_dk(const Problem &p, const PrefillArgs &a, const Segment &sg, hipStream_t st)
{
    switch (p.d_v) {
    case 32: return prepare_dv<DK, 32>(p, a, sg, st);
    case 64: return prepare_dv<DK, 64>(p, a, sg, st);
    case 128: return prepare_dv<DK, 128>(p, a, sg, st);
    }
    return hipErrorInvalidValue;
}

template <int DK, int DV>
hipError_t scan_dv(const Problem &p, const PrefillArgs &a, const Segment &sg, hipStream_t st)
{
    // with the epilogue the scan writes fp32 o (staged or in place)
    const bool ob = p.out_bf16 && !p.z;
    if (op_split(p))        // the prologue's two-term operands; z is then set or not
        return ob ? scan_t<DK, DV, bf16_t, bf16_t, true>(p, a, sg, st) : scan_t<DK, DV, bf16_t, float, true>(p, a, sg, st);
    if (op_bf16(p))
        return ob ? scan_t<DK, DV, bf16_t, bf16_t, false>(p, a, sg, st) : scan_t<DK, DV, bf16_t, float, false>(p, a, sg, st);
    return ob ? scan_t<DK, DV, float, bf16_t, false>(p, a, sg, st) : scan_t<DK, DV, float, float, false>(p, a, sg, st);
}

template <int DK>
hipError_t scan_dk(const Problem &p, const PrefillArgs &a, const Segment &sg, hipStream_t st)
{
    switch (p.d_v) {
    case 32: return scan_dv<DK, 32>(p, a, sg, st);
    case 64: return scan_dv<DK, 64>(p, a, sg, st);
    case 128: return scan_dv<DK, 128>(p, a, sg, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t prefill_workspace_bytes(const Problem &p, int32_t n_seqs, int64_t total_tokens, int slots)
{
    return ws_layout(p, n_seqs, total_tokens, slots).total;
}

int prefill_chunk_count(const Problem &p, int32_t n_seqs, int64_t total_tokens)
{
    return chunk_count(n_seqs, total_tokens);
}

int segment_chunks(const Problem &p, int chunks)
{
    const bool bf = op_bf16(p), si = op_split(p);
    const size_t per = (size_t)p.H_v * vblk_kib(p.d_k, p.d_v, bf, si) * 1024 +
                       (size_t)p.H_k * kblk_kib(p.d_k, bf, si) * 1024;
    if ((size_t)chunks * per <= kOneRangeBytes) return std::max(chunks, 1);
    const int fit = (int)std::max<size_t>(1, std::min<size_t>(kSegmentBytes / per, 0x7fffffff));
    // whole rounds of the preparation grid (chunks x key heads over its
    // workgroup slots), so that no range ends on a nearly empty round
    const int slots = (bf && !p.conv_w ? 2 : 1) * cu_count();
    const int round = std::max(1, slots / p.H_k);
    return fit >= round ? fit / round * round : fit;
}

hipError_t launch_prepare(const Problem &p, const PrefillArgs &a, const Segment &sg, hipStream_t st)
{
    switch (p.d_k) {
    case 32: return prepare_dk<32>(p, a, sg, st);
    case 64: return prepare_dk<64>(p, a, sg, st);
    case 128: return prepare_dk<128>(p, a, sg, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_scan(const Problem &p, const PrefillArgs &a, const Segment &sg, hipStream_t st)
{
    switch (p.d_k) {
    case 32: return scan_dk<32>(p, a, sg, st);
    case 64: return scan_dk<64>(p, a, sg, st);
    case 128: return scan_dk<128>(p, a, sg, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
