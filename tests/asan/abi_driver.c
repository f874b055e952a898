/*
 * Host-side driver of the libgdn C ABI for the AddressSanitizer build
 * (tests/test_host_asan.py).  It calls every entry point on paths that end
 * before any kernel launch: argument validation, workspace sizing, status
 * strings, the error message, the debug-record accessor and the environment
 * switches.  No GPU is needed.  Exit status: 0 when every call returned the
 * expected status; AddressSanitizer aborts the process on a memory error.
 */
#define _POSIX_C_SOURCE 200112L   /* setenv, unsetenv */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gdn.h"

static int failures = 0;

static void expect(const char *what, int got, int want)
{
    if (got != want) {
        fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, got, want, gdn_last_error());
        ++failures;
    }
}

static gdn_dims qwen(void)
{
    gdn_dims d;
    memset(&d, 0, sizeof d);
    d.H_k = 16;
    d.H_v = 32;
    d.d_k = 128;
    d.d_v = 128;
    d.dtype = GDN_BF16;
    d.eps = 1e-6f;
    return d;
}

int main(void)
{
    /* fake device addresses: never dereferenced on these paths */
    void *F = (void *)(uintptr_t)0x10000000u;
    float *Ff = (float *)F;
    int32_t *Fi = (int32_t *)F;
    size_t ws = 0;

    if (gdn_version() != GDN_VERSION) ++failures;
    for (int s = -3; s < 12; ++s)
        if (!gdn_status_string(s) || !gdn_status_string(s)[0]) ++failures;
    if (!gdn_last_error()) ++failures;

    /* sizing */
    gdn_dims d = qwen();
    expect("workspace 4096", gdn_prefill_workspace_size(&d, 1, 4096, &ws), GDN_OK);
    if (ws == 0 || ws % 256) ++failures;
    expect("chunked workspace 65536", gdn_chunked_prefill_workspace_size(&d, 1, 65536, &ws), GDN_OK);
    expect("workspace, 5000 sequences", gdn_prefill_workspace_size(&d, 5000, 12221, &ws), GDN_OK);
    expect("workspace, null dims", gdn_prefill_workspace_size(NULL, 1, 64, &ws), GDN_ERR_INVALID_ARG);
    expect("workspace, null out", gdn_prefill_workspace_size(&d, 1, 64, NULL), GDN_ERR_INVALID_ARG);
    expect("workspace, negative T", gdn_prefill_workspace_size(&d, 1, -5, &ws), GDN_ERR_INVALID_ARG);
    gdn_dims bad = qwen();
    bad.d_k = 96;
    expect("unsupported d_k", gdn_prefill_workspace_size(&bad, 1, 64, &ws), GDN_ERR_UNSUPPORTED);
    bad = qwen();
    bad.H_v = 24;
    bad.H_k = 16;
    expect("H_v not a multiple of H_k", gdn_prefill_workspace_size(&bad, 1, 64, &ws), GDN_ERR_UNSUPPORTED);
    bad = qwen();
    bad.d_conv = 4;
    expect("prologue without taps", gdn_prefill_workspace_size(&bad, 1, 64, &ws), GDN_ERR_INVALID_ARG);

    /* prefill argument validation (rejected before anything is enqueued) */
    expect("prefill, null q",
           gdn_chunked_prefill(&d, NULL, F, F, Ff, Ff, Ff, Ff, F, Fi, Fi, Fi, 1, 64, F, (size_t)1 << 40, NULL),
           GDN_ERR_INVALID_ARG);
    expect("prefill, small workspace",
           gdn_chunked_prefill(&d, F, F, F, Ff, Ff, Ff, Ff, F, Fi, Fi, Fi, 1, 64, F, 16, NULL),
           GDN_ERR_WORKSPACE);
    expect("prefill, misaligned out",
           gdn_chunked_prefill(&d, F, F, F, Ff, Ff, Ff, Ff, (char *)F + 2, Fi, Fi, Fi, 1, 64, F, (size_t)1 << 40, NULL),
           GDN_ERR_INVALID_ARG);
    expect("noalloc, null beta",
           gdn_chunked_prefill_noalloc(&d, F, F, F, Ff, NULL, Ff, Ff, F, Fi, Fi, Fi, 1, 64, NULL),
           GDN_ERR_INVALID_ARG);
    expect("prepare, zero sequences",
           gdn_prefill_prepare(&d, F, F, F, Ff, Ff, Fi, 0, 64, F, (size_t)1 << 40, NULL), GDN_ERR_INVALID_ARG);
    expect("scan, null state_out",
           gdn_prefill_scan(&d, Ff, NULL, F, Fi, Fi, 1, 64, F, (size_t)1 << 40, NULL), GDN_ERR_INVALID_ARG);
    expect("step, zero sequences",
           gdn_recurrent_step(&d, F, F, F, Ff, Ff, Ff, Ff, F, Fi, Fi, 0, NULL), GDN_ERR_INVALID_ARG);
    expect("multi, null cu_seqlens",
           gdn_recurrent_multi(&d, F, F, F, Ff, Ff, Ff, Ff, F, NULL, Fi, Fi, 4, 16, NULL), GDN_ERR_INVALID_ARG);
    bad = qwen();
    bad.d_conv = 4;
    bad.conv_w = Ff;
    expect("prologue with k given",
           gdn_recurrent_step(&bad, F, F, F, Ff, Ff, Ff, Ff, F, Fi, Fi, 4, NULL), GDN_ERR_INVALID_ARG);

    /* the error message survives long inputs */
    bad = qwen();
    bad.H_k = 2000000000;
    bad.H_v = 2000000000;
    (void)gdn_prefill_workspace_size(&bad, 2000000000, (int64_t)1 << 62, &ws);
    if (strlen(gdn_last_error()) >= 512) ++failures;

    /* debug record: nothing recorded in this process */
    gdn_debug_chunk rec;
    expect("debug dump, null", gdn_debug_dump(NULL), GDN_ERR_INVALID_ARG);
    expect("debug dump, none yet", gdn_debug_dump(&rec), GDN_ERR_INVALID_ARG);

    /* environment switches with malformed values: validation still comes first */
    const char *vals[] = {"", "x", "12", "1,", ",2", "-1,3", "3,-1", "99999999999999999999,1", "1,2,3",
                          "1 ,2", "7,7 ", NULL};
    for (int i = 0; vals[i]; ++i) {
        setenv("GDN_DEBUG_DUMP", vals[i], 1);
        setenv("GDN_CHECK", vals[i], 1);
        expect("prefill with switches, null q",
               gdn_chunked_prefill(&d, NULL, F, F, Ff, Ff, Ff, Ff, F, Fi, Fi, Fi, 1, 64, F, (size_t)1 << 40, NULL),
               GDN_ERR_INVALID_ARG);
    }
    unsetenv("GDN_DEBUG_DUMP");
    unsetenv("GDN_CHECK");

    if (failures) fprintf(stderr, "%d unexpected results\n", failures);
    else printf("abi driver: all host paths as expected\n");
    return failures ? 1 : 0;
}
