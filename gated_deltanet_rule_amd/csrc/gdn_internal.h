// gdn_internal.h -- launch interfaces between the C ABI (gdn_api.cpp) and the
// kernel translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

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
};

struct DecodeArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    const float *state_in;     // may be null: every sequence starts at zero
    float *state_out;
    void *out;
    const int32_t *slot_in, *slot_out;
    int32_t n_seqs;
};

hipError_t launch_decode(const Problem &p, const DecodeArgs &a, hipStream_t s);

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
};

// Chunk size of the WY form.
constexpr int kChunk = 64;

// Upper bound on the number of 64-token chunks of a packed batch.
inline int64_t max_chunks(int32_t n_seqs, int64_t total_tokens) {
    int64_t a = (total_tokens + kChunk - 1) / kChunk + n_seqs;
    return a;
}

size_t prefill_workspace_bytes(const Problem &p, int32_t n_seqs, int64_t total_tokens);
// state-independent phase: chunk table + per-chunk WY factors into the workspace
hipError_t launch_prepare(const Problem &p, const PrefillArgs &a, hipStream_t s);
// sequential phase: reads the workspace written by launch_prepare
hipError_t launch_scan(const Problem &p, const PrefillArgs &a, hipStream_t s);

}  // namespace gdn
