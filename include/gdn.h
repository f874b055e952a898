/*
 * gdn.h -- libgdn: the gated DeltaNet linear-attention operator on MI355X
 * (gfx950), behind a C ABI.
 *
 * The operator (per sequence and value head h; key head kh = h / (H_v/H_k)):
 *
 *     q^ = q / sqrt(|q|^2 + eps) * scale,   k^ = k / sqrt(|k|^2 + eps)
 *     S' = exp(g) * S                                   (decay first)
 *     delta = beta * (v - S'^T k^)                      (delta rule)
 *     S  = S' + k^ (x) delta                            (rank-1 correction)
 *     o  = S^T q^                                       (read-out, updated S)
 *
 * as built by the autoregressive graph on the page "Optimization: Qwen3 next
 * autoregressive pass (#17996)" (build_delta_net_autoregressive in
 * src/models/qwen3next.cpp), with q/k L2-normalised and q scaled by
 * 1/sqrt(head dim) as in both graphs there, and the key-head sharing of
 * "ik_llama.cpp src/llama-delta-net.cpp" (build_layer_attn_linear_core: with
 * the Qwen3-Next layout each key head is repeated H_v/H_k times in a row).
 * The state S is d_k x d_v fp32, stored row-major with d_v contiguous.
 *
 * Two entry points follow that page's split of the work (build_layer_attn_linear
 * chooses the autoregressive graph when a sequence brings one token and the
 * chunked graph otherwise):
 *   gdn_chunked_prefill  -- any number of tokens per sequence, chunked (64)
 *                           WY form on matrix cores (build_delta_net_chunking);
 *   gdn_recurrent_step   -- exactly one token per sequence;
 *   gdn_recurrent_multi  -- a few tokens per sequence, recurrent form.
 * State slots follow build_layer_attn_linear_core of the ik_llama.cpp page: the
 * state is read from a per-sequence slot (or starts at zero when the sequence
 * starts) and the new state is written back into a slot.
 *
 * Conventions for every call:
 *   - All tensor arguments are DEVICE pointers, contiguous, 16-byte aligned.
 *   - Layouts (T = total tokens; for gdn_recurrent_step T = n_seqs):
 *       q, k       [T][H_k][d_k]   element type dims->dtype
 *       v          [T][H_v][d_v]   element type dims->dtype
 *       out        [T][H_v][d_v]   element type dims->out_dtype
 *       g, beta    [T][H_v]        fp32; g is the log-decay (<= 0 expected),
 *                                  beta the post-sigmoid write strength
 *       state pools fp32, slot s at element offset s * slot_stride, inside a
 *                  slot [H_v][d_k][d_v]
 *       cu_seqlens [n_seqs+1] int32 device; sequence i owns tokens
 *                  [cu_seqlens[i], cu_seqlens[i+1]); cu_seqlens[0] == 0,
 *                  non-decreasing, cu_seqlens[n_seqs] == total_tokens
 *       slot_in, slot_out [n_seqs] int32 device; slot_in[i] < 0 means the
 *                  sequence starts from the zero state, slot_out[i] < 0
 *                  that its final state is not stored
 *   - The caller owns every buffer.  No call allocates, frees, synchronises
 *     or reads device memory on the host.  Work is enqueued on `stream`
 *     (a hipStream_t; NULL is the default stream) and completes
 *     asynchronously; nothing is retained after return.
 *   - Aliasing: state_out may equal state_in and slot_out[i] may equal
 *     slot_in[i] (in-place update).  Output slots must be distinct, and no
 *     sequence may write a slot that another sequence of the same call
 *     reads.  q/k/v/g/beta/out must not overlap the state pools or the
 *     workspace.
 *   - Errors: host-checkable arguments are validated before anything is
 *     enqueued; on error nothing is enqueued and a status != GDN_OK is
 *     returned, with a message from gdn_last_error().  Device-resident
 *     preconditions (cu_seqlens starting at 0, non-decreasing and ending at
 *     total_tokens; slot indices in range; distinct output slots; no output
 *     slot read by another sequence) are the caller's duty.  The kernels
 *     clamp sequence bounds into [0, total_tokens], so bad cu_seqlens give
 *     wrong results, not out-of-range accesses; a slot index outside the
 *     pool addresses memory outside it.  With the environment variable
 *     GDN_CHECK=1 every call first validates them on the device (one small
 *     kernel), waits for the result (a stream synchronisation: a debugging
 *     aid, not for timed or captured code) and returns GDN_ERR_INVALID_ARG,
 *     enqueueing nothing else, if one fails.  Each checked call reads its
 *     verdict from a word of its own (64 words per device, taken in turn:
 *     up to 64 checked calls may be in flight on one device at once, from
 *     any number of host threads).  Slot indices are checked for
 *     distinctness and aliasing (for up to 16384 sequences per call) and,
 *     when dims->n_slots > 0, against the pool size.  The library never
 *     aborts or throws.
 *   - Thread safety: calls may be made from several host threads; the error
 *     message is thread-local.
 *   - Graph capture: a call enqueues kernels only (no allocation, memset or
 *     synchronisation), so it may be captured into a HIP graph and replayed
 *     (with GDN_CHECK=1 or GDN_DEBUG_DUMP set a call synchronises and cannot
 *     be captured).
 *   - Debugging: GDN_DEBUG_DUMP=<token>,<head> makes the chunked prefill
 *     record the intermediates of one chunk (see gdn_debug_dump).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_VERSION 6

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = 1,   /* null pointer, bad count, bad alignment  */
    GDN_ERR_UNSUPPORTED = 2,   /* head dims / head ratio / dtype not built */
    GDN_ERR_WORKSPACE = 3,     /* workspace missing or too small           */
    GDN_ERR_HIP = 4            /* the HIP runtime reported an error        */
} gdn_status;

typedef enum gdn_dtype {
    GDN_F32 = 0,               /* fp32                                      */
    GDN_BF16 = 1               /* bfloat16                                  */
} gdn_dtype;

/*
 * Gate inputs.  GDN_GATES_FINAL: g is the log-decay and beta the write
 * strength, as the operator consumes them.  GDN_GATES_RAW: the g and beta
 * arguments carry the layer's raw projections a and b ([T][H_v] fp32) and the
 * kernels apply the activations of build_layer_attn_linear on the page
 * "Optimization: Qwen3 next autoregressive pass (#17996)" themselves:
 *     beta = sigmoid(b),    g = softplus(a + ssm_dt[h]) * ssm_a[h]
 * (softplus(x) = log(1 + e^x)), so the two small activation passes over
 * [T][H_v] never run.
 */
typedef enum gdn_gate_mode {
    GDN_GATES_FINAL = 0,
    GDN_GATES_RAW = 1
} gdn_gate_mode;

/*
 * Layer fusion (optional), the steps next to the operator in
 * build_layer_attn_linear_core on the page "ik_llama.cpp
 * src/llama-delta-net.cpp":
 *
 * Prologue (d_conv = 4): ggml_ssm_conv + ggml_silu.  The `q` argument of an
 * entry point then carries the mixed projection rows qkv [T][conv_dim]
 * (dims->dtype, conv_dim = 2*H_k*d_k + H_v*d_v, channels q | k | v in that
 * order) and `k`, `v` must be NULL.  Per channel c, with u the channel's d_conv-1
 * state values (oldest first) followed by the sequence's rows,
 *     x[t][c] = silu(sum_j conv_w[c][j] * u[t + j]),   silu(y) = y / (1 + e^-y),
 * and q, k, v are the three channel ranges of x.  The convolution state lives
 * at the start of every slot row of the state pools: a slot row is
 *     [conv_dim][d_conv-1] fp32 convolution state (oldest first), then
 *     [H_v][d_k][d_v] fp32 recurrent state,
 * so slot_stride (0 = the sum of both) and the state_in / state_out pointers
 * refer to whole rows.  slot_in < 0 starts both parts at zero; the new
 * convolution state (the last d_conv-1 inputs of u) is written at slot_out.
 * The convolution output is never rounded once to bf16 (after SiLU the keys
 * of neighbouring tokens are correlated, and a single bf16 rounding of q, k,
 * v moves the result by several percent of its rms): the recurrent entry
 * points use it in fp32, and with bf16 rows gdn_chunked_prefill feeds it to
 * the matrix cores as two-term bf16 operands (hi + lo, about 16 significant
 * bits; fp32 rows keep fp32 operands).  The prefill workspace grows
 * accordingly (the workspace sizes account for it).
 * The split-phase entry points do not support the prologue.
 *
 * Epilogue (z != NULL): llm_build_norm (RMS, weight ssm_norm) followed by
 * ggml_fused_mul_unary(z, ., SILU): each (token, value head) row o of the
 * operator's output becomes
 *     out = o / sqrt(mean(o^2) + eps) * norm_w * silu(z)
 * with the eps of the L2 norms.  gdn_recurrent_step and gdn_recurrent_multi
 * apply it before o leaves the chip; the chunked prefill applies it in a
 * pass after the scan, over fp32 o (in place in an fp32 `out`; with a bf16
 * `out`, o is staged in the workspace, which then grows by
 * 4*T*H_v*d_v bytes), so the result is rounded once.
 */

/* Problem dimensions shared by every entry point. */
typedef struct gdn_dims {
    int32_t H_k;          /* key heads (q and k)                            */
    int32_t H_v;          /* value heads; H_v % H_k == 0                    */
    int32_t d_k;          /* key head dim: 32, 64 or 128                    */
    int32_t d_v;          /* value head dim: 32, 64 or 128                  */
    int32_t dtype;        /* gdn_dtype of q, k and v                        */
    int32_t out_dtype;    /* gdn_dtype of out; GDN_F32 (0) matches the
                             pages' graphs, whose result is fp32; GDN_BF16
                             halves the output traffic at the cost of one
                             bf16 rounding per output element              */
    int64_t slot_stride;  /* elements between state slots; 0 means
                             H_v*d_k*d_v; else >= that and a multiple of 4  */
    float scale;          /* q scale; 0 means 1/sqrt(d_k)                   */
    float eps;            /* L2-norm epsilon, >= 0 (1e-6 for Qwen3-Next)    */
    int32_t gate_mode;    /* gdn_gate_mode: what the g and beta arguments
                             hold                                           */
    const float *ssm_a;   /* [H_v] device, fp32: per-value-head decay rate
                             (<= 0); read only with GDN_GATES_RAW          */
    const float *ssm_dt;  /* [H_v] device, fp32: per-value-head gate bias;
                             read only with GDN_GATES_RAW                   */
    int32_t d_conv;       /* 0: no prologue; 4: fused convolution prologue  */
    const float *conv_w;  /* [conv_dim][d_conv] device fp32, 16-byte
                             aligned, oldest tap first (with d_conv = 4)   */
    const void *z;        /* NULL: no epilogue; else the gate [T][H_v][d_v]
                             (dims->dtype), 16-byte aligned                */
    const float *norm_w;  /* [d_v] device fp32 RMS-norm weight (with z),
                             16-byte aligned                                */
    int32_t n_slots;      /* slots in the state pools (0: not given).  With
                             n_slots > 0, GDN_CHECK=1 also rejects a call
                             with slot_in[i] >= n_slots or
                             slot_out[i] >= n_slots; the kernels never read
                             it                                             */
} gdn_dims;

/* Library version (GDN_VERSION). */
int gdn_version(void);

/* Static description of a status code. */
const char *gdn_status_string(int status);

/* Detail of the last error raised on the calling thread ("" if none). */
const char *gdn_last_error(void);

/*
 * Workspace needed by the split-phase calls (gdn_prefill_prepare and
 * gdn_prefill_scan) for a batch of n_seqs sequences and total_tokens tokens,
 * written to *bytes; enough for gdn_chunked_prefill too.  Host-only, no
 * device work.  The workspace holds the chunk table and the per-chunk WY
 * factors (build_delta_net_chunking: k_cumdecay, the beta-weighted values and
 * the decayed q.k attention, plus q and k in matrix-core operand order)
 * between the two phases, one slot per chunk of the batch.
 */
gdn_status gdn_prefill_workspace_size(const gdn_dims *dims, int32_t n_seqs,
                                      int64_t total_tokens, size_t *bytes);

/*
 * Workspace needed by gdn_chunked_prefill for the same batch, written to
 * *bytes; at most gdn_prefill_workspace_size's.  Host-only, no device work
 * (it reads the current device's compute-unit count, 256 when there is no
 * device).  gdn_chunked_prefill runs a batch whose factors outgrow the GPU's
 * 256 MB last-level cache as consecutive ranges of chunks (preparation, then
 * scan, per range; results are bitwise those of one range); every range
 * writes its factors to the same slots, so the workspace holds one range's
 * factors (about 165 MiB at Qwen3-Next heads, against 2.6 GB for all of a
 * 65 536-token call's chunks), and a sequence that crosses a range boundary
 * keeps its state in one of two H_v x d_k x d_v fp32 carry states in between
 * (consecutive ranges use them in turn; at most one sequence crosses each
 * boundary).
 */
gdn_status gdn_chunked_prefill_workspace_size(const gdn_dims *dims, int32_t n_seqs,
                                              int64_t total_tokens, size_t *bytes);

/*
 * Chunked prefill: runs every sequence of a packed varlen batch through the
 * operator in chunks of 64 tokens (build_delta_net_chunking on the
 * "Optimization: Qwen3 next autoregressive pass (#17996)" page: cumulative
 * log-decay, the strictly lower beta*(k k^T)*decay matrix, (I+A)^-1, the WY
 * factors, intra-chunk attention and the inter-chunk state contribution;
 * a final partial chunk acts as if padded with identity rows).
 *
 *   q, k, v, g, beta : inputs, layouts above, total_tokens rows
 *   state_in         : fp32 slot pool read at slot_in[i] (may be NULL when
 *                      every slot_in[i] < 0)
 *   state_out        : fp32 slot pool written at slot_out[i]
 *   out              : [total_tokens][H_v][d_v] output, dims->out_dtype
 *   cu_seqlens       : [n_seqs+1] int32 (device)
 *   slot_in/slot_out : [n_seqs] int32 (device)
 *   n_seqs >= 1, total_tokens >= 0 (0: only the state pass-through runs)
 *   workspace        : device buffer of at least the size reported by
 *                      gdn_chunked_prefill_workspace_size (that of
 *                      gdn_prefill_workspace_size also serves), 256-byte
 *                      aligned
 * A zero-length sequence copies its input state (or zeros) to its out slot.
 */
gdn_status gdn_chunked_prefill(const gdn_dims *dims,
                               const void *q, const void *k, const void *v,
                               const float *g, const float *beta,
                               const float *state_in, float *state_out,
                               void *out, const int32_t *cu_seqlens,
                               const int32_t *slot_in, const int32_t *slot_out,
                               int32_t n_seqs, int64_t total_tokens,
                               void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * gdn_chunked_prefill without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It allocates nothing: its workspace is a
 * 64 MiB device array inside the library (each GPU the library runs on holds
 * its own copy until the process ends), and a batch whose factors outgrow it
 * runs as more, shorter chunk ranges (results are bitwise those of
 * gdn_chunked_prefill).  A batch that needs more than 64 MiB even in ranges
 * of one chunk (for example many thousands of sequences, or the epilogue
 * with a bf16 out, which stages 4*T*H_v*d_v bytes of fp32 output) is
 * rejected with GDN_ERR_WORKSPACE before anything is enqueued.  Every call
 * on one GPU uses that GPU's array, which keeps the last call's contents (no
 * call relies on them): calls that overlap on one GPU, from several streams
 * or host threads, race on it and must be ordered by the caller.  Other
 * arguments, layouts and errors as for gdn_chunked_prefill.
 */
gdn_status gdn_chunked_prefill_noalloc(const gdn_dims *dims,
                                       const void *q, const void *k, const void *v,
                                       const float *g, const float *beta,
                                       const float *state_in, float *state_out,
                                       void *out, const int32_t *cu_seqlens,
                                       const int32_t *slot_in, const int32_t *slot_out,
                                       int32_t n_seqs, int64_t total_tokens,
                                       void *stream);

/*
 * The two phases of gdn_chunked_prefill, for callers that schedule them
 * separately (for example, preparing ubatch n+1 on a second stream while the
 * scan of ubatch n runs; the scan is sequential over a sequence's chunks,
 * the preparation is not).  gdn_chunked_prefill(...) is exactly
 * gdn_prefill_prepare(...) followed by gdn_prefill_scan(...) on one stream.
 *
 * gdn_prefill_prepare: everything that does not depend on the carried state
 * (build_delta_net_chunking: g_cumsum, decay_mask, the beta*(k k^T)*decay
 * matrix and its triangular solve, k_cumdecay, the beta-weighted values
 * ("value" = T diag(beta) V) and the decayed q.k attention), written into
 * `workspace` together with the chunk table built from cu_seqlens (with
 * n_seqs == 1 no table is built: cu_seqlens is [0, total_tokens] by contract
 * and the chunks follow from total_tokens).  Reads q, k, v, g, beta and, for
 * n_seqs > 1, cu_seqlens.
 *
 * gdn_prefill_scan: the state-dependent part (v_prime / v_new, attn_inter +
 * v_attn, and the chunk-end state update), chunk after chunk per sequence,
 * reading only the workspace left by a prepare call with the same dims,
 * n_seqs and total_tokens (the caller orders the two, e.g. on one stream or
 * with an event) and the state pool; writes out and the state pool.
 * Arguments, layouts and errors as for gdn_chunked_prefill.
 */
gdn_status gdn_prefill_prepare(const gdn_dims *dims, const void *q, const void *k,
                               const void *v, const float *g, const float *beta,
                               const int32_t *cu_seqlens, int32_t n_seqs,
                               int64_t total_tokens, void *workspace,
                               size_t workspace_bytes, void *stream);

gdn_status gdn_prefill_scan(const gdn_dims *dims, const float *state_in, float *state_out,
                            void *out, const int32_t *slot_in, const int32_t *slot_out,
                            int32_t n_seqs, int64_t total_tokens, const void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * One autoregressive step: exactly one token for each of n_seqs sequences
 * (build_delta_net_autoregressive, which asserts a single token).  Token i
 * belongs to sequence i: q/k [n_seqs][H_k][d_k], v/out [n_seqs][H_v][d_v],
 * g/beta [n_seqs][H_v].  Reads state_in at slot_in[i] (zero state if < 0)
 * and writes state_out at slot_out[i].  Needs no workspace.
 */
gdn_status gdn_recurrent_step(const gdn_dims *dims,
                              const void *q, const void *k, const void *v,
                              const float *g, const float *beta,
                              const float *state_in, float *state_out,
                              void *out, const int32_t *slot_in,
                              const int32_t *slot_out, int32_t n_seqs,
                              void *stream);

/*
 * Debug record of the chunked form: the intermediates of one 64-token chunk
 * and one value head as the kernels computed them, for comparison with a
 * chunked reference.  They are the quantities of build_delta_net_chunking on
 * the page "Optimization: Qwen3 next autoregressive pass (#17996)":
 * g_cumsum (G), the solved and unit-diagonal attn (T = (I + A)^-1 with
 * A = strict_lower(diag(beta) k^ k^T * decay_mask)), k_cumdecay
 * (W = T diag(beta e^G) k^) and v_new (U = T diag(beta) v - W S, S the state
 * entering the chunk).
 *
 * With the environment variable GDN_DEBUG_DUMP=<token>,<head> (packed token
 * index and value head, both >= 0), gdn_chunked_prefill and the pair
 * gdn_prefill_prepare / gdn_prefill_scan record the chunk holding that token
 * for that head: the preparation writes G, T and W, the scan U, into a
 * device buffer the library allocates once per device; the call that ends
 * the prefill (gdn_chunked_prefill, or gdn_prefill_scan) then synchronises
 * its stream and copies the record to the host.  A call whose batch does not
 * reach the token leaves `prepared` and `scanned` at 0.  A debugging aid:
 * such calls allocate (once), synchronise and cannot be captured, and calls
 * that overlap in time share the record.  gdn_chunked_prefill_noalloc
 * ignores the variable.  Rows at or past `len` and columns at or past d_k
 * (W) or d_v (U) are unspecified.
 */
typedef struct gdn_debug_chunk {
    int32_t token, head;      /* as requested                                   */
    int32_t chunk;            /* index of the chunk within the batch            */
    int32_t t0, len;          /* its packed tokens [t0, t0 + len)               */
    int32_t d_k, d_v;
    int32_t prepared;         /* 1: G, T and W were written                     */
    int32_t scanned;          /* 1: U was written                               */
    int32_t reserved;
    double G[64];             /* cumulative log-decay within the chunk          */
    float T[64][64];          /* row-major                                      */
    float W[64][128];         /* token rows, d_k columns                        */
    float U[64][128];         /* token rows, d_v columns                        */
} gdn_debug_chunk;

/* Copy the last debug record into *out (host memory).  GDN_ERR_INVALID_ARG
 * when out is NULL or no prefill has run with GDN_DEBUG_DUMP set. */
gdn_status gdn_debug_dump(gdn_debug_chunk *out);

/*
 * Several tokens per sequence in the recurrent form: the single-chunk case
 * the page "Optimization: Qwen3 next autoregressive pass (#17996)" removed
 * from build_layer_attn_linear (build_delta_net_recurrent, used when a
 * sequence brings at most one chunk), here for short multi-token batches such
 * as speculative-decoding verification.  Same arguments, layouts and slot
 * semantics as gdn_chunked_prefill (tokens packed by cu_seqlens), no
 * workspace.  The tokens of a sequence are processed one after the other with
 * the state block in registers: each state is read and written once per call,
 * and the work per token is that of gdn_recurrent_step.  Correct for any
 * length; for sequences longer than about one chunk gdn_chunked_prefill is
 * faster.  Empty sequences pass their state through (zero if slot_in < 0).
 */
gdn_status gdn_recurrent_multi(const gdn_dims *dims,
                               const void *q, const void *k, const void *v,
                               const float *g, const float *beta,
                               const float *state_in, float *state_out,
                               void *out, const int32_t *cu_seqlens,
                               const int32_t *slot_in, const int32_t *slot_out,
                               int32_t n_seqs, int64_t total_tokens,
                               void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
