// gdn_api.cpp -- the libgdn C ABI: argument validation, workspace sizing and
// dispatch to the kernel launchers.  No allocation, no synchronisation and no
// host reads of device memory happen here, except in the two debugging modes
// (GDN_CHECK, GDN_DEBUG_DUMP).
#include <algorithm>
#include <mutex>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/gdn.h"
#include "gdn_internal.h"

namespace {

thread_local char g_last_error[512] = "";

gdn_status fail(gdn_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_dim(int d) { return d == 32 || d == 64 || d == 128; }

gdn_status resolve(const gdn_dims *d, gdn::Problem *p)
{
    if (!d) return fail(GDN_ERR_INVALID_ARG, "dims is NULL");
    if (d->H_k <= 0 || d->H_v <= 0)
        return fail(GDN_ERR_INVALID_ARG, "head counts must be positive (H_k=%d, H_v=%d)", d->H_k, d->H_v);
    if (d->H_v % d->H_k != 0)
        return fail(GDN_ERR_UNSUPPORTED, "H_v (%d) must be a multiple of H_k (%d)", d->H_v, d->H_k);
    if (!supported_dim(d->d_k) || !supported_dim(d->d_v))
        return fail(GDN_ERR_UNSUPPORTED, "head dims must be 32, 64 or 128 (d_k=%d, d_v=%d)", d->d_k, d->d_v);
    if (d->dtype != GDN_F32 && d->dtype != GDN_BF16)
        return fail(GDN_ERR_UNSUPPORTED, "unknown dtype %d", d->dtype);
    if (d->out_dtype != GDN_F32 && d->out_dtype != GDN_BF16)
        return fail(GDN_ERR_UNSUPPORTED, "unknown out_dtype %d", d->out_dtype);
    if (d->d_conv != 0 && d->d_conv != gdn::kConv)
        return fail(GDN_ERR_UNSUPPORTED, "d_conv must be 0 or %d (got %d)", gdn::kConv, d->d_conv);
    const int64_t conv_dim = 2 * (int64_t)d->H_k * d->d_k + (int64_t)d->H_v * d->d_v;
    if (conv_dim > INT32_MAX / gdn::kConv) return fail(GDN_ERR_UNSUPPORTED, "too many channels");
    const int64_t conv_state = d->d_conv ? (gdn::kConv - 1) * conv_dim : 0;
    const int64_t slot = conv_state + (int64_t)d->H_v * d->d_k * d->d_v;
    int64_t stride = d->slot_stride == 0 ? slot : d->slot_stride;
    if (stride < slot || stride % 4 != 0)
        return fail(GDN_ERR_INVALID_ARG, "slot_stride %lld must be 0 or a multiple of 4 >= %lld",
                    (long long)d->slot_stride, (long long)slot);
    if (!(d->eps >= 0.f) || !isfinite(d->eps)) return fail(GDN_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (!(d->scale >= 0.f) || !isfinite(d->scale)) return fail(GDN_ERR_INVALID_ARG, "scale must be finite and >= 0");
    p->H_k = d->H_k;
    p->H_v = d->H_v;
    p->d_k = d->d_k;
    p->d_v = d->d_v;
    p->bf16 = d->dtype == GDN_BF16;
    p->out_bf16 = d->out_dtype == GDN_BF16;
    p->slot_stride = stride;
    p->scale = d->scale == 0.f ? 1.0f / sqrtf((float)d->d_k) : d->scale;
    p->eps = d->eps;
    if (d->gate_mode != GDN_GATES_FINAL && d->gate_mode != GDN_GATES_RAW)
        return fail(GDN_ERR_INVALID_ARG, "unknown gate_mode %d", d->gate_mode);
    p->ssm_a = p->ssm_dt = nullptr;
    if (d->gate_mode == GDN_GATES_RAW) {
        if (!d->ssm_a || !d->ssm_dt)
            return fail(GDN_ERR_INVALID_ARG, "GDN_GATES_RAW needs ssm_a and ssm_dt");
        if (!aligned(d->ssm_a, 4) || !aligned(d->ssm_dt, 4))
            return fail(GDN_ERR_INVALID_ARG, "ssm_a / ssm_dt are not 4-byte aligned");
        p->ssm_a = d->ssm_a;
        p->ssm_dt = d->ssm_dt;
    }
    p->conv_dim = (int)conv_dim;
    p->conv_state = conv_state;
    p->conv_w = nullptr;
    if (d->d_conv) {
        if (!d->conv_w) return fail(GDN_ERR_INVALID_ARG, "d_conv = %d needs conv_w", d->d_conv);
        if (!aligned(d->conv_w, 16)) return fail(GDN_ERR_INVALID_ARG, "conv_w is not 16-byte aligned");
        p->conv_w = d->conv_w;
    }
    p->rs_qk = d->d_conv ? conv_dim : (int64_t)d->H_k * d->d_k;
    p->rs_v = d->d_conv ? conv_dim : (int64_t)d->H_v * d->d_v;
    if (d->n_slots < 0) return fail(GDN_ERR_INVALID_ARG, "n_slots must be >= 0 (got %d)", d->n_slots);
    p->n_slots = d->n_slots;
    p->z = d->z;
    p->norm_w = nullptr;
    if (d->z) {
        if (!aligned(d->z, 16)) return fail(GDN_ERR_INVALID_ARG, "z is not 16-byte aligned");
        if (!d->norm_w) return fail(GDN_ERR_INVALID_ARG, "the epilogue (z) needs norm_w");
        if (!aligned(d->norm_w, 16)) return fail(GDN_ERR_INVALID_ARG, "norm_w is not 16-byte aligned");
        p->norm_w = d->norm_w;
    }
    return GDN_OK;
}

// With the prologue, `q` carries the mixed rows and k, v are its channel
// ranges; the caller must leave k and v NULL.
gdn_status mixed_rows(const gdn::Problem &p, const void *&q, const void *&k, const void *&v)
{
    if (!p.conv_w) return GDN_OK;
    if (k || v) return fail(GDN_ERR_INVALID_ARG, "with d_conv, q carries the mixed q|k|v rows: k and v must be NULL");
    if (!q) return fail(GDN_ERR_INVALID_ARG, "q (the mixed rows) is NULL");
    const size_t es = p.bf16 ? 2 : 4;
    const char *b = static_cast<const char *>(q);
    k = b + es * (size_t)p.H_k * p.d_k;
    v = b + es * 2 * (size_t)p.H_k * p.d_k;
    return GDN_OK;
}

// The recurrent part of a slot row follows its convolution state.
const float *ssm_part(const gdn::Problem &p, const float *s) { return s ? s + p.conv_state : nullptr; }
float *ssm_part(const gdn::Problem &p, float *s) { return s ? s + p.conv_state : nullptr; }

gdn_status hip_status(hipError_t e, const char *what)
{
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
    return GDN_OK;
}

// GDN_CHECK=1: validate the device-side preconditions before any kernel of
// the call is launched (synchronises `s`; debugging aid, not for timing).
bool check_mode()
{
    const char *e = getenv("GDN_CHECK");
    return e && e[0] == '1' && e[1] == 0;
}

// GDN_DEBUG_DUMP=<token>,<head>: the prefill records one chunk's
// intermediates (gdn_debug_dump).  The device record is allocated once per
// device and kept until the process ends; the last host copy is shared by
// every thread.
constexpr int kMaxDevices = 64;
std::mutex g_dbg_mu;
gdn_debug_chunk *g_dbg_dev[kMaxDevices] = {};
gdn_debug_chunk g_dbg_last;
bool g_dbg_have = false;

bool debug_target(int *token, int *head)
{
    const char *e = getenv("GDN_DEBUG_DUMP");
    if (!e || !*e) return false;
    char extra;
    return sscanf(e, "%d,%d%c", token, head, &extra) == 2 && *token >= 0 && *head >= 0;
}

// Attach the device record to `p` when the variable is set; `clear` marks it
// unwritten (the call that runs the preparation).
gdn_status debug_setup(gdn::Problem &p, hipStream_t s, bool clear)
{
    int token, head;
    if (!debug_target(&token, &head)) return GDN_OK;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "GDN_DEBUG_DUMP: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(GDN_ERR_UNSUPPORTED, "GDN_DEBUG_DUMP: device %d", dev);
    {
        std::lock_guard<std::mutex> lk(g_dbg_mu);
        if (!g_dbg_dev[dev]) {
            e = hipMalloc(reinterpret_cast<void **>(&g_dbg_dev[dev]), sizeof(gdn_debug_chunk));
            if (e != hipSuccess) {
                g_dbg_dev[dev] = nullptr;
                return fail(GDN_ERR_HIP, "GDN_DEBUG_DUMP: %s", hipGetErrorString(e));
            }
        }
    }
    p.dbg = g_dbg_dev[dev];
    p.dbg_token = token;
    p.dbg_head = head;
    // all-ones: chunk -1 and the written flags -1 until a kernel sets them
    if (clear) e = hipMemsetAsync(p.dbg, 0xff, sizeof(gdn_debug_chunk), s);
    return e == hipSuccess ? GDN_OK : fail(GDN_ERR_HIP, "GDN_DEBUG_DUMP: %s", hipGetErrorString(e));
}

// After the scan: wait for the stream and keep a host copy of the record.
gdn_status debug_collect(const gdn::Problem &p, hipStream_t s)
{
    if (!p.dbg) return GDN_OK;
    gdn_debug_chunk rec;
    hipError_t e = hipMemcpyAsync(&rec, p.dbg, sizeof rec, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "GDN_DEBUG_DUMP: %s", hipGetErrorString(e));
    rec.token = p.dbg_token;
    rec.head = p.dbg_head;
    rec.d_k = p.d_k;
    rec.d_v = p.d_v;
    rec.reserved = 0;
    if (rec.prepared != 1) {
        rec.prepared = 0;
        rec.chunk = -1;
        rec.t0 = rec.len = 0;
    }
    if (rec.scanned != 1) rec.scanned = 0;
    std::lock_guard<std::mutex> lk(g_dbg_mu);
    g_dbg_last = rec;
    g_dbg_have = true;
    return GDN_OK;
}

gdn_status device_check(const gdn::Problem &p, const int32_t *cu, int32_t n, int64_t T,
                        const int32_t *slot_in, const int32_t *slot_out, hipStream_t s)
{
    if (!check_mode()) return GDN_OK;
    int v = 0;
    gdn_status st = hip_status(gdn::run_check(cu, n, T, slot_in, slot_out, p.n_slots, s, &v),
                               "GDN_CHECK validation");
    if (st != GDN_OK) return st;
    if (v & gdn::kCheckCuStart) return fail(GDN_ERR_INVALID_ARG, "GDN_CHECK: cu_seqlens[0] is not 0");
    if (v & gdn::kCheckCuEnd)
        return fail(GDN_ERR_INVALID_ARG, "GDN_CHECK: cu_seqlens[n_seqs] differs from total_tokens (%lld)",
                    (long long)T);
    if (v & gdn::kCheckCuOrder) return fail(GDN_ERR_INVALID_ARG, "GDN_CHECK: cu_seqlens is not non-decreasing");
    if (v & gdn::kCheckSlotDup) return fail(GDN_ERR_INVALID_ARG, "GDN_CHECK: two sequences write the same slot");
    if (v & gdn::kCheckSlotAlias)
        return fail(GDN_ERR_INVALID_ARG, "GDN_CHECK: a sequence writes a slot that another sequence reads");
    if (v & gdn::kCheckSlotRange)
        return fail(GDN_ERR_INVALID_ARG, "GDN_CHECK: a slot index is not below n_slots (%d)", p.n_slots);
    return GDN_OK;
}

gdn_status check_tensors(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *state_in, float *state_out,
                         void *out, const int32_t *slot_in, const int32_t *slot_out)
{
    struct { const void *p; const char *name; size_t align; } t[] = {
        {q, "q", 16}, {k, "k", 16}, {v, "v", 16}, {g, "g", 4}, {beta, "beta", 4},
        {state_out, "state_out", 16}, {out, "out", 16}, {slot_in, "slot_in", 4},
        {slot_out, "slot_out", 4}};
    for (auto &e : t) {
        if (!e.p) return fail(GDN_ERR_INVALID_ARG, "%s is NULL", e.name);
        if (!aligned(e.p, e.align))
            return fail(GDN_ERR_INVALID_ARG, "%s is not %zu-byte aligned", e.name, e.align);
    }
    if (state_in && !aligned(state_in, 16)) return fail(GDN_ERR_INVALID_ARG, "state_in is not 16-byte aligned");
    return GDN_OK;
}

gdn_status check_counts(int32_t n_seqs, int64_t total_tokens)
{
    if (n_seqs < 1) return fail(GDN_ERR_INVALID_ARG, "n_seqs must be >= 1 (got %d)", n_seqs);
    if (n_seqs > (1 << 24)) return fail(GDN_ERR_UNSUPPORTED, "n_seqs above 16M");
    if (total_tokens < 0 || total_tokens > INT32_MAX)
        return fail(GDN_ERR_INVALID_ARG, "total_tokens out of range (%lld)", (long long)total_tokens);
    return GDN_OK;
}

gdn_status check_workspace(const gdn::Problem &p, int32_t n_seqs, int64_t total_tokens,
                           const void *workspace, size_t workspace_bytes, int slots = 0)
{
    const size_t need = gdn::prefill_workspace_bytes(p, n_seqs, total_tokens, slots);
    if (!workspace || workspace_bytes < need)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu at %p)", need,
                    workspace_bytes, workspace);
    if (!aligned(workspace, 256)) return fail(GDN_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    return GDN_OK;
}

gdn_status check_prepare_inputs(const void *q, const void *k, const void *v, const float *g,
                                const float *beta, const int32_t *cu_seqlens)
{
    struct { const void *p; const char *name; size_t align; } t[] = {
        {q, "q", 16}, {k, "k", 16}, {v, "v", 16}, {g, "g", 4}, {beta, "beta", 4},
        {cu_seqlens, "cu_seqlens", 4}};
    for (auto &e : t) {
        if (!e.p) return fail(GDN_ERR_INVALID_ARG, "%s is NULL", e.name);
        if (!aligned(e.p, e.align))
            return fail(GDN_ERR_INVALID_ARG, "%s is not %zu-byte aligned", e.name, e.align);
    }
    return GDN_OK;
}

gdn_status check_scan_inputs(const float *state_in, float *state_out, void *out,
                             const int32_t *slot_in, const int32_t *slot_out)
{
    struct { const void *p; const char *name; size_t align; } t[] = {
        {state_out, "state_out", 16}, {out, "out", 16}, {slot_in, "slot_in", 4},
        {slot_out, "slot_out", 4}};
    for (auto &e : t) {
        if (!e.p) return fail(GDN_ERR_INVALID_ARG, "%s is NULL", e.name);
        if (!aligned(e.p, e.align))
            return fail(GDN_ERR_INVALID_ARG, "%s is not %zu-byte aligned", e.name, e.align);
    }
    if (state_in && !aligned(state_in, 16)) return fail(GDN_ERR_INVALID_ARG, "state_in is not 16-byte aligned");
    return GDN_OK;
}

// The chunked prefill of a validated call: device check, then `per`-chunk
// ranges (preparation, scan) over the workspace, then the convolution state.
gdn_status run_chunked(gdn::Problem p, const void *q, const void *k,
                       const void *v, const float *g, const float *beta, const float *state_in,
                       float *state_out, void *out, const int32_t *cu_seqlens,
                       const int32_t *slot_in, const int32_t *slot_out, int32_t n_seqs,
                       int64_t total_tokens, void *workspace, int per, hipStream_t s,
                       bool debug = true)
{
    if (p.H_v > 65535) return fail(GDN_ERR_UNSUPPORTED, "H_v above 65535");
    const int chunks = gdn::prefill_chunk_count(p, n_seqs, total_tokens);
    const int n_seg = std::max(1, (chunks + per - 1) / per);
    gdn::PrefillArgs a{q, k, v, g, beta, ssm_part(p, state_in), ssm_part(p, state_out), out,
                       cu_seqlens, slot_in, slot_out, n_seqs, total_tokens, workspace,
                       state_in, state_out, per};
    gdn_status st = device_check(p, cu_seqlens, n_seqs, total_tokens, slot_in, slot_out, s);
    if (st == GDN_OK && debug) st = debug_setup(p, s, true);
    if (st != GDN_OK) return st;
    for (int r = 0; r < n_seg && st == GDN_OK; ++r) {
        gdn::Segment sg;
        sg.lo = r * per;
        sg.hi = r + 1 == n_seg ? 0x7fffffff : (r + 1) * per;
        sg.idx = r;
        sg.first = r == 0;
        sg.last = r + 1 == n_seg;
        st = hip_status(gdn::launch_prepare(p, a, sg, s), "prepare");
        if (st == GDN_OK) st = hip_status(gdn::launch_scan(p, a, sg, s), "scan");
    }
    // (with the prologue the scans also replace each sequence's convolution
    // state, in the range that holds its last chunk)
    if (st == GDN_OK) st = debug_collect(p, s);
    return st;
}

}  // namespace

extern "C" {

int gdn_version(void) { return GDN_VERSION; }

gdn_status gdn_debug_dump(gdn_debug_chunk *out)
{
    g_last_error[0] = 0;
    if (!out) return fail(GDN_ERR_INVALID_ARG, "gdn_debug_dump: out is NULL");
    std::lock_guard<std::mutex> lk(g_dbg_mu);
    if (!g_dbg_have) return fail(GDN_ERR_INVALID_ARG, "gdn_debug_dump: no prefill has run with GDN_DEBUG_DUMP set");
    *out = g_dbg_last;
    return GDN_OK;
}

const char *gdn_status_string(int status)
{
    switch (status) {
    case GDN_OK: return "success";
    case GDN_ERR_INVALID_ARG: return "invalid argument";
    case GDN_ERR_UNSUPPORTED: return "unsupported configuration";
    case GDN_ERR_WORKSPACE: return "workspace missing or too small";
    case GDN_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *gdn_last_error(void) { return g_last_error; }

gdn_status gdn_prefill_workspace_size(const gdn_dims *dims, int32_t n_seqs,
                                      int64_t total_tokens, size_t *bytes)
{
    g_last_error[0] = 0;
    gdn::Problem p;
    gdn_status st = resolve(dims, &p);
    if (st != GDN_OK) return st;
    if (!bytes) return fail(GDN_ERR_INVALID_ARG, "bytes is NULL");
    if (n_seqs < 1) return fail(GDN_ERR_INVALID_ARG, "n_seqs must be >= 1 (got %d)", n_seqs);
    if (total_tokens < 0 || total_tokens > INT32_MAX)
        return fail(GDN_ERR_INVALID_ARG, "total_tokens out of range (%lld)", (long long)total_tokens);
    *bytes = gdn::prefill_workspace_bytes(p, n_seqs, total_tokens);
    return GDN_OK;
}

gdn_status gdn_chunked_prefill_workspace_size(const gdn_dims *dims, int32_t n_seqs,
                                              int64_t total_tokens, size_t *bytes)
{
    g_last_error[0] = 0;
    gdn::Problem p;
    gdn_status st = resolve(dims, &p);
    if (st != GDN_OK) return st;
    if (!bytes) return fail(GDN_ERR_INVALID_ARG, "bytes is NULL");
    st = check_counts(n_seqs, total_tokens);
    if (st != GDN_OK) return st;
    const int per = gdn::segment_chunks(p, gdn::prefill_chunk_count(p, n_seqs, total_tokens));
    *bytes = gdn::prefill_workspace_bytes(p, n_seqs, total_tokens, per);
    return GDN_OK;
}

gdn_status gdn_prefill_prepare(const gdn_dims *dims, const void *q, const void *k,
                               const void *v, const float *g, const float *beta,
                               const int32_t *cu_seqlens, int32_t n_seqs, int64_t total_tokens,
                               void *workspace, size_t workspace_bytes, void *stream)
{
    g_last_error[0] = 0;
    gdn::Problem p;
    gdn_status st = resolve(dims, &p);
    if (st == GDN_OK && p.conv_w)
        st = fail(GDN_ERR_UNSUPPORTED, "the convolution prologue reads the slot state: use gdn_chunked_prefill");
    if (st == GDN_OK) st = check_counts(n_seqs, total_tokens);
    if (st == GDN_OK) st = check_prepare_inputs(q, k, v, g, beta, cu_seqlens);
    if (st == GDN_OK) st = check_workspace(p, n_seqs, total_tokens, workspace, workspace_bytes);
    if (st != GDN_OK) return st;
    st = device_check(p, cu_seqlens, n_seqs, total_tokens, nullptr, nullptr, static_cast<hipStream_t>(stream));
    if (st == GDN_OK) st = debug_setup(p, static_cast<hipStream_t>(stream), true);
    if (st != GDN_OK) return st;
    gdn::PrefillArgs a{q, k, v, g, beta, nullptr, nullptr, nullptr, cu_seqlens, nullptr,
                       nullptr, n_seqs, total_tokens, workspace, nullptr, nullptr};
    return hip_status(gdn::launch_prepare(p, a, gdn::Segment{}, static_cast<hipStream_t>(stream)), "prepare");
}

gdn_status gdn_prefill_scan(const gdn_dims *dims, const float *state_in, float *state_out,
                            void *out, const int32_t *slot_in, const int32_t *slot_out,
                            int32_t n_seqs, int64_t total_tokens, const void *workspace,
                            size_t workspace_bytes, void *stream)
{
    g_last_error[0] = 0;
    gdn::Problem p;
    gdn_status st = resolve(dims, &p);
    if (st == GDN_OK && p.conv_w)
        st = fail(GDN_ERR_UNSUPPORTED, "the convolution prologue reads the slot state: use gdn_chunked_prefill");
    if (st == GDN_OK) st = check_counts(n_seqs, total_tokens);
    if (st == GDN_OK) st = check_scan_inputs(state_in, state_out, out, slot_in, slot_out);
    if (st == GDN_OK) st = check_workspace(p, n_seqs, total_tokens, workspace, workspace_bytes);
    if (st != GDN_OK) return st;
    if (p.H_v > 65535) return fail(GDN_ERR_UNSUPPORTED, "H_v above 65535");
    gdn::PrefillArgs a{nullptr, nullptr, nullptr, nullptr, nullptr, state_in, state_out, out, nullptr, slot_in,
                       slot_out, n_seqs, total_tokens, const_cast<void *>(workspace), nullptr, nullptr};
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = device_check(p, nullptr, n_seqs, n_seqs, slot_in, slot_out, s);
    if (st == GDN_OK) st = debug_setup(p, s, false);
    if (st != GDN_OK) return st;
    st = hip_status(gdn::launch_scan(p, a, gdn::Segment{}, s), "scan");
    if (st == GDN_OK) st = debug_collect(p, s);
    return st;
}

gdn_status gdn_chunked_prefill(const gdn_dims *dims, const void *q, const void *k,
                               const void *v, const float *g, const float *beta,
                               const float *state_in, float *state_out, void *out,
                               const int32_t *cu_seqlens, const int32_t *slot_in,
                               const int32_t *slot_out, int32_t n_seqs,
                               int64_t total_tokens, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    g_last_error[0] = 0;
    gdn::Problem p;
    gdn_status st = resolve(dims, &p);
    if (st == GDN_OK) st = mixed_rows(p, q, k, v);
    if (st == GDN_OK) st = check_counts(n_seqs, total_tokens);
    if (st == GDN_OK) st = check_prepare_inputs(q, k, v, g, beta, cu_seqlens);
    if (st == GDN_OK) st = check_scan_inputs(state_in, state_out, out, slot_in, slot_out);
    if (st != GDN_OK) return st;
    // consecutive chunk ranges within the cache budget, each writing its
    // factors to the same per chunk slots
    const int chunks = gdn::prefill_chunk_count(p, n_seqs, total_tokens);
    const int per = gdn::segment_chunks(p, chunks);
    st = check_workspace(p, n_seqs, total_tokens, workspace, workspace_bytes, per);
    if (st != GDN_OK) return st;
    return run_chunked(p, q, k, v, g, beta, state_in, state_out, out, cu_seqlens, slot_in,
                       slot_out, n_seqs, total_tokens, workspace, per, static_cast<hipStream_t>(stream));
}

gdn_status gdn_chunked_prefill_noalloc(const gdn_dims *dims, const void *q, const void *k,
                                       const void *v, const float *g, const float *beta,
                                       const float *state_in, float *state_out, void *out,
                                       const int32_t *cu_seqlens, const int32_t *slot_in,
                                       const int32_t *slot_out, int32_t n_seqs,
                                       int64_t total_tokens, void *stream)
{
    g_last_error[0] = 0;
    gdn::Problem p;
    gdn_status st = resolve(dims, &p);
    if (st == GDN_OK) st = mixed_rows(p, q, k, v);
    if (st == GDN_OK) st = check_counts(n_seqs, total_tokens);
    if (st == GDN_OK) st = check_prepare_inputs(q, k, v, g, beta, cu_seqlens);
    if (st == GDN_OK) st = check_scan_inputs(state_in, state_out, out, slot_in, slot_out);
    if (st != GDN_OK) return st;
    void *ws = nullptr;
    size_t cap = 0;
    st = hip_status(gdn::scratch_buffer(&ws, &cap), "scratch lookup");
    if (st != GDN_OK) return st;
    // the longest chunk range (at most the one gdn_chunked_prefill would
    // use) whose workspace fits the scratch: the size is monotone in it
    const int chunks = gdn::prefill_chunk_count(p, n_seqs, total_tokens);
    int lo = 1, hi = gdn::segment_chunks(p, chunks);
    const size_t need1 = gdn::prefill_workspace_bytes(p, n_seqs, total_tokens, lo);
    if (need1 > cap)
        return fail(GDN_ERR_WORKSPACE,
                    "gdn_chunked_prefill_noalloc: this batch needs %zu bytes of scratch even in ranges "
                    "of one chunk; the allocation-free entry point holds %zu (use gdn_chunked_prefill)",
                    need1, cap);
    while (lo < hi) {
        const int mid = lo + (hi - lo + 1) / 2;
        if (gdn::prefill_workspace_bytes(p, n_seqs, total_tokens, mid) <= cap) lo = mid;
        else hi = mid - 1;
    }
    return run_chunked(p, q, k, v, g, beta, state_in, state_out, out, cu_seqlens, slot_in,
                       slot_out, n_seqs, total_tokens, ws, lo, static_cast<hipStream_t>(stream), false);
}

gdn_status gdn_recurrent_step(const gdn_dims *dims, const void *q, const void *k,
                              const void *v, const float *g, const float *beta,
                              const float *state_in, float *state_out, void *out,
                              const int32_t *slot_in, const int32_t *slot_out,
                              int32_t n_seqs, void *stream)
{
    g_last_error[0] = 0;
    gdn::Problem p;
    gdn_status st = resolve(dims, &p);
    if (st != GDN_OK) return st;
    if (n_seqs < 1) return fail(GDN_ERR_INVALID_ARG, "n_seqs must be >= 1 (got %d)", n_seqs);
    if (n_seqs > INT32_MAX / 2) return fail(GDN_ERR_UNSUPPORTED, "n_seqs too large");
    if (p.H_v > 65535) return fail(GDN_ERR_UNSUPPORTED, "H_v above 65535");
    const void *qkv = q;
    st = mixed_rows(p, q, k, v);
    if (st == GDN_OK) st = check_tensors(q, k, v, g, beta, state_in, state_out, out, slot_in, slot_out);
    if (st != GDN_OK) return st;
    gdn::DecodeArgs a{q, k, v, g, beta, ssm_part(p, state_in), ssm_part(p, state_out), out,
                      slot_in, slot_out, n_seqs, state_in, state_out};
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = device_check(p, nullptr, n_seqs, n_seqs, slot_in, slot_out, s);
    if (st != GDN_OK) return st;
    st = hip_status(gdn::launch_decode(p, a, s), "decode");
    if (st == GDN_OK && p.conv_w && !gdn::decode_folds_conv(p))
        st = hip_status(gdn::launch_conv_state(p, qkv, nullptr, -1, n_seqs, n_seqs, state_in, state_out,
                                               slot_in, slot_out, s), "convolution state");
    return st;
}

gdn_status gdn_recurrent_multi(const gdn_dims *dims, const void *q, const void *k,
                               const void *v, const float *g, const float *beta,
                               const float *state_in, float *state_out, void *out,
                               const int32_t *cu_seqlens, const int32_t *slot_in,
                               const int32_t *slot_out, int32_t n_seqs,
                               int64_t total_tokens, void *stream)
{
    g_last_error[0] = 0;
    gdn::Problem p;
    gdn_status st = resolve(dims, &p);
    const void *qkv = q;
    if (st == GDN_OK) st = mixed_rows(p, q, k, v);
    if (st == GDN_OK) st = check_counts(n_seqs, total_tokens);
    if (st == GDN_OK) st = check_prepare_inputs(q, k, v, g, beta, cu_seqlens);
    if (st == GDN_OK) st = check_scan_inputs(state_in, state_out, out, slot_in, slot_out);
    if (st != GDN_OK) return st;
    if (n_seqs > 0x7fffffff / 2) return fail(GDN_ERR_UNSUPPORTED, "n_seqs too large");
    if (p.H_v > 65535) return fail(GDN_ERR_UNSUPPORTED, "H_v above 65535");
    gdn::DecodeMultiArgs a{q, k, v, g, beta, ssm_part(p, state_in), ssm_part(p, state_out), out,
                           cu_seqlens, slot_in, slot_out, n_seqs, total_tokens, state_in, state_out};
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = device_check(p, cu_seqlens, n_seqs, total_tokens, slot_in, slot_out, s);
    if (st != GDN_OK) return st;
    st = hip_status(gdn::launch_decode_multi(p, a, s), "multi-token decode");
    if (st == GDN_OK && p.conv_w && !gdn::decode_folds_conv(p))
        st = hip_status(gdn::launch_conv_state(p, qkv, cu_seqlens, -1, n_seqs, total_tokens, state_in,
                                               state_out, slot_in, slot_out, s), "convolution state");
    return st;
}

}  // extern "C"
