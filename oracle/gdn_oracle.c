/*
 * gdn_oracle.c -- fp64 CPU oracle for the gated DeltaNet operator.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or constant with the
 * HIP library.
 *
 * Sources (the pages are cited by title and the function or passage used):
 *   [AR]  "Optimization: Qwen3 next autoregressive pass (#17996)", the new
 *         build_delta_net_autoregressive graph in src/models/qwen3next.cpp:
 *         decay the state by exp(g), kv_mem = sum over the key axis of
 *         state * k, delta = (v - kv_mem) * beta, state += k (x) delta, and
 *         the read-out sum over the key axis of state * q (taken from the
 *         updated state).
 *   [CH]  the same page, build_delta_net_chunking and the body of the removed
 *         build_delta_net_recurrent (the single-chunk WY form): cumulative
 *         log-decay, decay mask, the strictly lower beta*(k k^T)*decay matrix,
 *         its triangular solve, value / k_cumdecay, v_prime, v_new,
 *         attn_inter, the chunk-end state update.
 *   [NORM] both graphs: q and k are L2-normalised (eps = f_norm_rms_eps) and
 *         q is scaled by 1/sqrt(head dim).
 *   [GQA] "ik_llama.cpp src/llama-delta-net.cpp", build_layer_attn_linear_core:
 *         with the Qwen3-Next (fused beta/alpha) layout each key head is
 *         repeated H_v/H_k times in a row, so value head h reads key head
 *         h / (H_v/H_k).
 *   [SLOT] same file, build_layer_attn_linear_core: the state is read from the
 *         sequence's slot (zeroed when the sequence starts) and the new state
 *         is copied back into a slot.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - L2 norm: x / sqrt(sum x^2 + eps) (the eps value is passed in).
 *   - scale passed in (1/sqrt(d_k) by default; d_k == d_v in every workload).
 *   - a partial final chunk is processed with its real rows only (equivalent
 *     to the pages' padding with identity rows).
 *
 * Pins (tests/test_oracle_pins.py): the T=1 closed form, beta=0 pure decay,
 * g=0/beta=1 orthonormal-key storage and overwrite, the O(T^2) materialised
 * form solved with a library triangular solver, chunked == sequential for
 * several chunk sizes, and the structural invariances (varlen packing, state
 * carry across calls, GQA duplication, affinity in S0, linearity in V, head
 * permutation).  Mutation tests re-compile this file with single plausible
 * mistakes planted and check that some pin fails.
 *
 * Layouts (all row-major, token-major, the same as the library's):
 *   q, k   [T][H_k][d_k]   fp64 (exact bf16 or fp32 inputs, or fp64 values
 *                           from the convolution prologue of oracle/layer.py)
 *   v      [T][H_v][d_v]   fp64, likewise
 *   g,beta [T][H_v]         fp64 (exact fp32 inputs, or fp64 values from the
 *                           gate activations of oracle/__init__.py)
 *   s0     [n_seqs][H_v][d_k][d_v] fp64 (NULL = zero state)
 *   out    [T][H_v][d_v]  fp64
 *   s_out  [n_seqs][H_v][d_k][d_v] fp64
 * Only the value heads listed in `heads` (all when NULL) are computed; the
 * other heads' outputs are left untouched.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t n_seqs;
    const int64_t *cu;
    int32_t H_k, H_v, d_k, d_v;
    const double *q, *k, *v;
    const double *g, *beta;
    const double *s0;
    double scale, eps;
    const int32_t *heads;
    int32_t n_heads;
    double *out, *s_out;
    int32_t chunk;          /* 0 = sequential recurrence, else chunk size */
    /* chunk record (gdn_oracle_chunk_dump): the intermediates of the chunk
       holding packed token dump_token for value head dump_head */
    int64_t dump_token;     /* < 0: none */
    int32_t dump_head;
    double *dump_G, *dump_T, *dump_W, *dump_U;   /* C, C x C, C x d_k, C x d_v */
    int64_t *dump_meta;     /* t0, n */
    int32_t n_threads;
    int32_t next;           /* work counter */
    pthread_mutex_t lock;
    int32_t status;
} job_t;

/* [NORM] x_hat = x / sqrt(sum(x^2) + eps), times an extra factor */
static void l2_normalise(const double *x, int n, double eps, double factor, double *y)
{
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += x[i] * x[i];
    double inv = factor / sqrt(ss + eps);
    for (int i = 0; i < n; ++i) y[i] = x[i] * inv;
}

/* One (sequence, value head) chain, token by token: [AR]. */
static void run_sequential(const job_t *J, int s, int h, double *S,
                           double *qh, double *kh, double *kv)
{
    const int dk = J->d_k, dv = J->d_v;
    const int r = J->H_v / J->H_k;
    const int hk = h / r;                                   /* [GQA] */
    for (int64_t t = J->cu[s]; t < J->cu[s + 1]; ++t) {
        l2_normalise(J->q + (t * J->H_k + hk) * dk, dk, J->eps, J->scale, qh);
        l2_normalise(J->k + (t * J->H_k + hk) * dk, dk, J->eps, 1.0, kh);
        const double a = exp(J->g[t * J->H_v + h]);
        const double b = J->beta[t * J->H_v + h];
        const double *vt = J->v + (t * J->H_v + h) * dv;
        /* decay first */
        for (int i = 0; i < dk * dv; ++i) S[i] *= a;
        /* kv_mem[j] = sum_i S[i][j] k[i]  (from the decayed state) */
        for (int j = 0; j < dv; ++j) kv[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) kv[j] += S[i * dv + j] * kh[i];
        /* delta = beta (v - kv_mem); S += k (x) delta */
        for (int j = 0; j < dv; ++j) kv[j] = b * ((double)vt[j] - kv[j]);
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[i * dv + j] += kh[i] * kv[j];
        /* o[j] = sum_i S[i][j] q[i]  (from the updated state) */
        double *o = J->out + (t * J->H_v + h) * dv;
        for (int j = 0; j < dv; ++j) o[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) o[j] += S[i * dv + j] * qh[i];
    }
}

/* One (sequence, value head) chain in the chunked WY form: [CH].
 * Per chunk of n <= C rows with incoming state S (d_k x d_v):
 *   G      = inclusive cumsum of g over the chunk
 *   decay  D[r][c] = exp(G[r] - G[c]) for c <= r, else 0 (masked before exp)
 *   attn   = -(beta_r k_r.k_c) D[r][c] for c < r  (strictly lower), call it -A
 *   solve (I + A) X = -A, then T = X (strict part) + I  (= (I + A)^-1)
 *   value      = T (beta V)
 *   k_cumdecay = T (beta exp(G) K)
 *   qk         = (q_r.k_c) D[r][c] for c <= r
 *   v_prime    = k_cumdecay S ;  v_new = value - v_prime
 *   attn_inter = (exp(G) Q) S ;  out = attn_inter + qk v_new
 *   S          = S exp(G[n-1]) + (K exp(G[n-1] - G))^T v_new
 */
static void run_chunked(const job_t *J, int s, int h, double *S, double *wk)
{
    const int dk = J->d_k, dv = J->d_v, C = J->chunk;
    const int r = J->H_v / J->H_k;
    const int hk = h / r;
    double *Q = wk;                  /* C x dk */
    double *K = Q + (size_t)C * dk;  /* C x dk */
    double *V = K + (size_t)C * dk;  /* C x dv */
    double *G = V + (size_t)C * dv;  /* C */
    double *B = G + C;               /* C (beta) */
    double *D = B + C;               /* C x C decay mask */
    double *M = D + (size_t)C * C;   /* C x C: -A, then T */
    double *X = M + (size_t)C * C;   /* C x C solve result */
    double *VAL = X + (size_t)C * C; /* C x dv value */
    double *KCD = VAL + (size_t)C * dv; /* C x dk k_cumdecay */
    double *QK = KCD + (size_t)C * dk;  /* C x C */
    double *VN = QK + (size_t)C * C;    /* C x dv v_new */

    for (int64_t t0 = J->cu[s]; t0 < J->cu[s + 1]; t0 += C) {
        int n = (int)((J->cu[s + 1] - t0) < C ? (J->cu[s + 1] - t0) : C);
        for (int a = 0; a < n; ++a) {
            int64_t t = t0 + a;
            l2_normalise(J->q + (t * J->H_k + hk) * dk, dk, J->eps, J->scale, Q + a * dk);
            l2_normalise(J->k + (t * J->H_k + hk) * dk, dk, J->eps, 1.0, K + a * dk);
            for (int j = 0; j < dv; ++j) V[a * dv + j] = J->v[(t * J->H_v + h) * dv + j];
            B[a] = J->beta[t * J->H_v + h];
            G[a] = (a ? G[a - 1] : 0.0) + J->g[t * J->H_v + h];
        }
        for (int a = 0; a < n; ++a)
            for (int c = 0; c < n; ++c)
                D[a * C + c] = (c <= a) ? exp(G[a] - G[c]) : 0.0;
        /* attn = -(k_beta k^T * decay) strictly lower */
        for (int a = 0; a < n; ++a)
            for (int c = 0; c < n; ++c) {
                double kk = 0.0;
                for (int i = 0; i < dk; ++i) kk += B[a] * K[a * dk + i] * K[c * dk + i];
                M[a * C + c] = (c < a) ? -(kk * D[a * C + c]) : 0.0;
            }
        /* (I - attn) X = attn by forward substitution (unit lower lhs) */
        for (int c = 0; c < n; ++c)
            for (int a = 0; a < n; ++a) {
                double acc = M[a * C + c];
                for (int m = 0; m < a; ++m) acc += M[a * C + m] * X[m * C + c];
                X[a * C + c] = acc;   /* lhs[a][m] = -M[a][m] for m < a */
            }
        /* T = strict_lower(X) + I */
        for (int a = 0; a < n; ++a)
            for (int c = 0; c < n; ++c)
                M[a * C + c] = (c < a) ? X[a * C + c] : (c == a ? 1.0 : 0.0);
        /* value = T (beta V);  k_cumdecay = T (beta exp(G) K) */
        for (int a = 0; a < n; ++a) {
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int c = 0; c < n; ++c) acc += M[a * C + c] * B[c] * V[c * dv + j];
                VAL[a * dv + j] = acc;
            }
            for (int i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int c = 0; c < n; ++c) acc += M[a * C + c] * B[c] * exp(G[c]) * K[c * dk + i];
                KCD[a * dk + i] = acc;
            }
        }
        /* qk = (q k^T) * decay, lower including the diagonal */
        for (int a = 0; a < n; ++a)
            for (int c = 0; c < n; ++c) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += Q[a * dk + i] * K[c * dk + i];
                QK[a * C + c] = (c <= a) ? acc * D[a * C + c] : 0.0;
            }
        /* v_new = value - k_cumdecay S */
        for (int a = 0; a < n; ++a)
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += KCD[a * dk + i] * S[i * dv + j];
                VN[a * dv + j] = VAL[a * dv + j] - acc;
            }
        /* chunk record: copies of g_cumsum, T, k_cumdecay and v_new */
        if (J->dump_token >= t0 && J->dump_token < t0 + n && h == J->dump_head) {
            for (int a = 0; a < n; ++a) {
                J->dump_G[a] = G[a];
                for (int c = 0; c < n; ++c) J->dump_T[a * C + c] = M[a * C + c];
                for (int i = 0; i < dk; ++i) J->dump_W[a * dk + i] = KCD[a * dk + i];
                for (int j = 0; j < dv; ++j) J->dump_U[a * dv + j] = VN[a * dv + j];
            }
            J->dump_meta[0] = t0;
            J->dump_meta[1] = n;
        }
        /* out = (exp(G) Q) S + qk v_new */
        for (int a = 0; a < n; ++a) {
            double *o = J->out + ((t0 + a) * J->H_v + h) * dv;
            double eg = exp(G[a]);
            for (int j = 0; j < dv; ++j) {
                double inter = 0.0, intra = 0.0;
                for (int i = 0; i < dk; ++i) inter += eg * Q[a * dk + i] * S[i * dv + j];
                for (int c = 0; c < n; ++c) intra += QK[a * C + c] * VN[c * dv + j];
                o[j] = inter + intra;
            }
        }
        /* S = S exp(G_last) + (K exp(G_last - G))^T v_new */
        double gl = G[n - 1];
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int c = 0; c < n; ++c) acc += K[c * dk + i] * exp(gl - G[c]) * VN[c * dv + j];
                S[i * dv + j] = S[i * dv + j] * exp(gl) + acc;
            }
    }
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const int dk = J->d_k, dv = J->d_v;
    const int nh = J->heads ? J->n_heads : J->H_v;
    const int64_t n_items = (int64_t)J->n_seqs * nh;
    size_t C = (size_t)(J->chunk > 0 ? J->chunk : 1);
    size_t wk_len = 2 * C * dk + 2 * C * dv + 2 * C + 4 * C * C + C * dk + C * dv + (size_t)dk + dk + dv;
    double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
    double *wk = (double *)malloc(sizeof(double) * wk_len);
    if (!S || !wk) {
        pthread_mutex_lock(&J->lock);
        J->status = -2;
        pthread_mutex_unlock(&J->lock);
        free(S); free(wk);
        return NULL;
    }
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t item = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (item >= n_items) break;
        int s = (int)(item / nh);
        int h = J->heads ? J->heads[item % nh] : (int)(item % nh);
        size_t soff = ((size_t)s * J->H_v + h) * dk * dv;
        if (J->s0) memcpy(S, J->s0 + soff, sizeof(double) * dk * dv);
        else memset(S, 0, sizeof(double) * dk * dv);           /* [SLOT] reset */
        if (J->chunk > 0) run_chunked(J, s, h, S, wk);
        else run_sequential(J, s, h, S, wk, wk + dk, wk + 2 * dk);
        memcpy(J->s_out + soff, S, sizeof(double) * dk * dv);
    }
    free(S);
    free(wk);
    return NULL;
}

static int run(job_t *J)
{
    if (J->n_seqs < 0 || J->H_k <= 0 || J->H_v <= 0 || J->d_k <= 0 || J->d_v <= 0) return -1;
    if (J->H_v % J->H_k != 0) return -1;
    if (J->heads) {
        for (int i = 0; i < J->n_heads; ++i)
            if (J->heads[i] < 0 || J->heads[i] >= J->H_v) return -1;
    }
    for (int s = 0; s < J->n_seqs; ++s)
        if (J->cu[s + 1] < J->cu[s]) return -1;
    int nt = J->n_threads > 0 ? J->n_threads : 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nt);
    if (!th) return -2;
    pthread_mutex_init(&J->lock, NULL);
    J->next = 0;
    J->status = 0;
    int started = 0;
    for (int i = 0; i < nt; ++i) {
        if (pthread_create(&th[i], NULL, worker, J) != 0) break;
        ++started;
    }
    if (started == 0) worker(J);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&J->lock);
    free(th);
    return J->status;
}

int gdn_oracle_run(int32_t n_seqs, const int64_t *cu_seqlens,
                   int32_t H_k, int32_t H_v, int32_t d_k, int32_t d_v,
                   const double *q, const double *k, const double *v,
                   const double *g, const double *beta, const double *s0,
                   double scale, double eps,
                   const int32_t *heads, int32_t n_heads,
                   double *out, double *s_out,
                   int32_t chunk, int32_t n_threads)
{
    job_t J;
    memset(&J, 0, sizeof J);
    J.n_seqs = n_seqs; J.cu = cu_seqlens;
    J.H_k = H_k; J.H_v = H_v; J.d_k = d_k; J.d_v = d_v;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.s0 = s0;
    J.scale = scale; J.eps = eps;
    J.heads = heads; J.n_heads = n_heads;
    J.out = out; J.s_out = s_out;
    J.chunk = chunk < 0 ? 0 : chunk;
    J.n_threads = n_threads;
    J.dump_token = -1;
    return run(&J);
}

/*
 * The chunked form (chunk size `chunk`) for value head `head` only, keeping
 * a copy of the intermediates of the chunk that holds packed token `token`:
 * G (g_cumsum, chunk entries), T (the solved attn plus identity, chunk x
 * chunk row-major), W (k_cumdecay, chunk x d_k) and U (v_new, chunk x d_v);
 * meta receives the chunk's first token and length (length 0: no chunk holds
 * the token).  out and s_out receive that head's results as gdn_oracle_run
 * gives them.
 */
int gdn_oracle_chunk_dump(int32_t n_seqs, const int64_t *cu_seqlens,
                          int32_t H_k, int32_t H_v, int32_t d_k, int32_t d_v,
                          const double *q, const double *k, const double *v,
                          const double *g, const double *beta, const double *s0,
                          double scale, double eps, int32_t chunk, int64_t token, int32_t head,
                          double *out, double *s_out,
                          double *G, double *T, double *W, double *U, int64_t *meta)
{
    if (chunk <= 0 || head < 0 || head >= H_v) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.n_seqs = n_seqs; J.cu = cu_seqlens;
    J.H_k = H_k; J.H_v = H_v; J.d_k = d_k; J.d_v = d_v;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.s0 = s0;
    J.scale = scale; J.eps = eps;
    J.heads = &head; J.n_heads = 1;
    J.out = out; J.s_out = s_out;
    J.chunk = chunk;
    J.n_threads = 1;
    J.dump_token = token; J.dump_head = head;
    J.dump_G = G; J.dump_T = T; J.dump_W = W; J.dump_U = U; J.dump_meta = meta;
    meta[0] = 0;
    meta[1] = 0;
    return run(&J);
}
