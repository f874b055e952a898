// gdn_internal.h -- launch interfaces between the C ABI (gdn_api.cpp) and the
// kernel translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

struct gdn_debug_chunk;   // include/gdn.h

namespace gdn {

// Validated, fully resolved problem description handed to the launchers.
struct Problem {
    int H_k, H_v, d_k, d_v;
    int bf16;              // 1: q/k/v are bfloat16, 0: fp32
    int out_bf16;          // 1: out is bfloat16, 0: fp32
    int64_t slot_stride;   // elements
    float scale, eps;
    // raw gates: beta = sigmoid(b), g = softplus(a + ssm_dt[h]) * ssm_a[h]
    const float *ssm_a;    // null: g and beta are given as the operator takes them
    const float *ssm_dt;
    // row strides (elements) of q / k and of v: H_k d_k and H_v d_v, or
    // conv_dim when the three are channel ranges of the mixed rows
    int64_t rs_qk, rs_v;
    // prologue: x = silu(causal conv(qkv)), convolution state at the start of
    // each slot row (conv_state floats); conv_w null = off
    const float *conv_w;   // [conv_dim][kConv]
    int conv_dim;
    int64_t conv_state;    // (kConv - 1) * conv_dim, 0 when off
    // epilogue: out = o / sqrt(mean(o^2) + eps) * norm_w * silu(z); z null = off
    const void *z;
    const float *norm_w;
    // slots in the state pools (0: unknown); read only by check mode
    int n_slots;
    // debug record (GDN_DEBUG_DUMP): null when off, else the device record of
    // the chunk holding packed token dbg_token, for value head dbg_head
    gdn_debug_chunk *dbg = nullptr;
    int dbg_token = -1, dbg_head = -1;
};

// Taps of the fused convolution prologue.
constexpr int kConv = 4;

// State pointers below address the recurrent state of slot 0; with the
// prologue, conv_in / conv_out address the slot rows themselves (the
// convolution state at their start).
struct DecodeArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    const float *state_in;     // may be null: every sequence starts at zero
    float *state_out;
    void *out;
    const int32_t *slot_in, *slot_out;
    int32_t n_seqs;
    const float *conv_in;
    float *conv_out;
};

hipError_t launch_decode(const Problem &p, const DecodeArgs &a, hipStream_t s);

// With the prologue and H_v / H_k in {1, 2} the recurrent kernels replace the
// convolution state themselves (one workgroup per (sequence, key head));
// otherwise the caller runs launch_conv_state after them.
bool decode_folds_conv(const Problem &p);

// several tokens per sequence, recurrent form, no workspace
struct DecodeMultiArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    const float *state_in;     // may be null: every sequence starts at zero
    float *state_out;
    void *out;
    const int32_t *cu_seqlens, *slot_in, *slot_out;
    int32_t n_seqs;
    int64_t total_tokens;
    const float *conv_in;
    float *conv_out;
};

hipError_t launch_decode_multi(const Problem &p, const DecodeMultiArgs &a, hipStream_t s);

struct PrefillArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    const float *state_in;
    float *state_out;
    void *out;
    const int32_t *cu_seqlens, *slot_in, *slot_out;
    int32_t n_seqs;
    int64_t total_tokens;
    void *workspace;
    const float *conv_in;
    float *conv_out;
    // WY-factor slots the workspace holds: 0 for one per chunk of the batch
    // (the split-phase calls), else the chunk-range length (gdn_chunked_prefill,
    // whose ranges reuse the slots of the first)
    int ws_slots = 0;
};

// Chunk size of the WY form.
constexpr int kChunk = 64;

// Upper bound on the number of 64-token chunks of a packed batch.
inline int64_t max_chunks(int32_t n_seqs, int64_t total_tokens) {
    int64_t a = (total_tokens + kChunk - 1) / kChunk + n_seqs;
    return a;
}

size_t prefill_workspace_bytes(const Problem &p, int32_t n_seqs, int64_t total_tokens, int slots = 0);

// A range of chunks run as one preparation + scan pair.  A long prefill is
// run as several consecutive ranges so that the WY factors one range writes
// are still in the 256 MB last-level cache (the MALL) when its scan reads
// them: once they outgrow it, the scan's time per chunk rises by half.
// Sequences crossing a range boundary carry their state through the
// workspace.
struct Segment {
    int lo = 0, hi = 0x7fffffff;   // chunks [lo, hi) of the batch
    int idx = 0;                   // index of the range
    bool first = true;             // the first range: builds the chunk table
    bool last = true;              // the last range: runs the epilogue
};
// A batch whose factors fit kOneRangeBytes runs as one range (a second
// launch pair costs more than the cache misses it saves); a longer one runs
// in ranges of at most kSegmentBytes of factors, which leaves room in the
// cache for the range's outputs.  Every range writes its factors to the same
// workspace slots (chunk c of the range at slot c - lo), so a range rewrites
// lines the cache already holds.  Measured at Qwen3-Next heads: 5120 tokens
// (206 MiB of factors) 163 us as one range against 186 us as two; 8192
// tokens 231 us in ranges of 64 chunks (165 MiB), 263 us in ranges of 32 and
// 289 us in ranges of 96; the fused layer's 4096 tokens (226 MiB) 294-300 us
// as two ranges against 345 us as one.
constexpr size_t kOneRangeBytes = 212u << 20;
constexpr size_t kSegmentBytes = 168u << 20;
// chunks of a batch (an upper bound when n_seqs > 1) and chunks per range
int prefill_chunk_count(const Problem &p, int32_t n_seqs, int64_t total_tokens);
int segment_chunks(const Problem &p, int chunks);
// state-independent phase: chunk table + per-chunk WY factors into the workspace
hipError_t launch_prepare(const Problem &p, const PrefillArgs &a, const Segment &sg, hipStream_t s);
// sequential phase: reads the workspace written by launch_prepare (and runs
// the gated RMSNorm epilogue when p.z is set)
hipError_t launch_scan(const Problem &p, const PrefillArgs &a, const Segment &sg, hipStream_t s);

// Allocation-free prefill (gdn_scratch.hip): the calling thread's current
// device's copy of a file-scope device array of kScratchBytes, 256-byte
// aligned, shared by every call on that device.
constexpr size_t kScratchBytes = 64u << 20;
hipError_t scratch_buffer(void **ptr, size_t *bytes);

// Check mode (GDN_CHECK=1, gdn_check.hip): validates cu_seqlens (null: one
// token per sequence) and the slot lists of a call on the device, then
// synchronises the stream and returns its findings, a set of these bits.
constexpr int kCheckCuStart = 1;     // cu_seqlens[0] != 0
constexpr int kCheckCuEnd = 2;       // cu_seqlens[n_seqs] != total_tokens
constexpr int kCheckCuOrder = 4;     // cu_seqlens decreases somewhere
constexpr int kCheckSlotDup = 8;     // two sequences write the same slot
constexpr int kCheckSlotAlias = 16;  // a sequence writes a slot another one reads
constexpr int kCheckSlotRange = 32;  // a slot index at or past n_slots (when given)
hipError_t run_check(const int32_t *cu, int32_t n, int64_t T, const int32_t *slot_in, const int32_t *slot_out,
                     int n_slots, hipStream_t s, int *flags);

// Layer fusion passes (gdn_layer.hip).
// New convolution state of every sequence: the last kConv - 1 inputs of its
// state followed by its rows.  `cu` null: sequence i is row i (one token
// each); single_T >= 0: one sequence of rows [0, single_T).  Runs after every
// reader of the old state (it may be written in place).
hipError_t launch_conv_state(const Problem &p, const void *qkv, const int32_t *cu, int single_T,
                             int32_t n_seqs, int64_t total_tokens, const float *conv_in,
                             float *conv_out, const int32_t *slot_in, const int32_t *slot_out,
                             hipStream_t s);
// Gated RMSNorm of the fp32 rows o (T x H_v rows of d_v) into `out`
// (out_dtype; may be o itself when that is fp32).
hipError_t launch_gated_norm(const Problem &p, const float *o, void *out, int64_t total_tokens, hipStream_t s);

}  // namespace gdn
