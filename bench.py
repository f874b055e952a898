#!/usr/bin/env python3
"""libgdn benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--quick]

Headline (`value`): chunked-prefill throughput in tokens/s on the single-layer
Qwen3-Next-shaped prefill (1 sequence, T=4096, H_k=16, H_v=32, d_k=d_v=128,
bf16 q/k/v, fp32 g/beta/state, fp32 output, chunk 64).  One step = one
gdn_prefill_prepare + gdn_prefill_scan over that batch (every prefill row of
the path), inputs resident in HBM.  The step first runs untimed for 100 ms so that the
GPU's clocks settle, then W untimed warm-up steps, then exactly K timed steps
between two device synchronisations.

Alongside (same JSON line):
  roofline      the prefill's dominant kernel, from HIP events recorded on the
                stream the kernels run on around K launches of that kernel
                back to back (after the timed steps): algorithmic flops per launch
                (per token per value head, split by the kernel that forms each
                product; see prefill_flops_per_token_head) / mean launch time,
                against the bf16 dense MFMA peak (2.5 PFLOP/s spec, and the
                peak measured on this GPU by libgdnpeak.so).
  prefill_step_roofline  the whole step: 8*C*d + 6*d^2 flops per token-head
                over ms_per_step, against both peaks.
  measured_peaks  bf16 MFMA throughput and HBM copy / read rates measured here.
  decode        gdn_recurrent_step on 64 sequences x 128 steps: tokens/s and
                state + I/O bytes / kernel time against the 8 TB/s HBM peak
                and the measured copy rate, headline from the ping-pong run
                (two 128 MiB pools, 256 MiB footprint, beyond the 256 MB
                last-level cache); the in-place run (128 MiB) alongside.
  decode_multi  gdn_recurrent_multi on 64 sequences x 4 tokens (speculative
                verification), state in place; HBM roofline on state + I/O.
  varlen        8 packed sequences of 17..8192 tokens (12221), one call.
  stream        65536 tokens as 128 calls of 512 with the state carried.
  layer_prefill the fused layer path (convolution prologue, raw gates, gated
                RMSNorm epilogue) on the T=4096 prefill, one call.
  layer_decode  the fused layer path on the decode workload, per step.
  layer_multi   the fused layer path on the 64 x 4 multi-token workload.
  cpu_baseline  the fp64 oracle (test infrastructure, never tuned) on the
                same prefill workload, on this host's cores.
The gates follow the workloads' recipe: beta = sigmoid(b) and
g = -exp(A_log) softplus(a) of the raw draws a, b ~ N(0, 1), evaluated here
(workload_gates).
All inputs are seeded synthetic data (see gdn_inputs.py).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gdn_inputs as gi  # noqa: E402

METRIC = "GDN prefill tokens/s (MFMA util) + decode tokens/s (state HBM GB/s), 1 GPU"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
C = 64

# HBM bytes per launch of the prefill kernels on the T=4096 workload: rocprofv3
# FETCH_SIZE and WRITE_SIZE (one run each, profiles/prefill_T4096_hbm_traffic.md),
# scaled by what the same counters read for a 256 MiB device copy (x2.000 and
# x1.000).  They hold only for the kernel source they were taken on; after any
# change to its code (comments aside) the bench reports traffic as null until
# the counters are retaken.
PREFILL_SRC = [os.path.join(ROOT, "gated_deltanet_rule_amd", "csrc", f)
               for f in ("gdn_prefill.hip", "gdn_mfma.h", "gdn_device.h", "gdn_internal.h")]
MEASURED_TRAFFIC = {
    "source_sha256": "ace15307f041711fe6d158b857305fad90c9139d6587a2901b9bea434f2d9615",
    "scan": (79541.0 * 2.000 + 67584.0 * 1.000) * 1024,
    "prepare": (34001.9 * 2.000 + 156741.0 * 1.000) * 1024,
}


# The same for the decode kernel on the 64 x 128 decode workload
# (profiles/decode64x128_hbm_traffic.md), per launch.
DECODE_SRC = [os.path.join(ROOT, "gated_deltanet_rule_amd", "csrc", f)
              for f in ("gdn_decode.hip", "gdn_device.h", "gdn_internal.h")]
MEASURED_DECODE_TRAFFIC = {
    "source_sha256": "63b31562283da88aa828759356d09f680d1bf501fc60011d736b3e4025747225",
    "decode": (66152.4 * 2.000 + 132096.0 * 1.000) * 1024,
}


def source_digest(paths):
    """SHA-256 of C/HIP sources with comments and blank space removed, so
    that edits to comments alone do not invalidate measurements."""
    import hashlib
    import re
    h = hashlib.sha256()
    for path in paths:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = "\n".join(line.strip() for line in text.splitlines() if line.strip())
        h.update(text.encode())
    return h.hexdigest()


def measured_traffic(kernel):
    if kernel == "decode":
        ok = source_digest(DECODE_SRC) == MEASURED_DECODE_TRAFFIC["source_sha256"]
        return MEASURED_DECODE_TRAFFIC["decode"] if ok else None
    ok = source_digest(PREFILL_SRC) == MEASURED_TRAFFIC["source_sha256"]
    return MEASURED_TRAFFIC.get(kernel) if ok else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def workload_gates(a, b, ssm_a, ssm_dt):
    """The workloads' gates from the generator's raw draws a, b ~ N(0, 1):
    beta = sigmoid(b), g = ssm_a * softplus(a + ssm_dt) (ssm_dt = 0 for the
    named workloads), evaluated in fp64 and rounded once to fp32."""
    x = np.asarray(a, np.float64) + np.asarray(ssm_dt, np.float64)[None, :]
    softplus = np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))
    bb = np.asarray(b, np.float64)
    e = np.exp(-np.abs(bb))
    beta = np.where(bb >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    g = softplus * np.asarray(ssm_a, np.float64)[None, :]
    return g.astype(np.float32), beta.astype(np.float32)


WG = dict(final_gates=workload_gates)


def prefill_flops_per_token_head(H_k, H_v, d_k, d_v):
    """Algorithmic flops per token per value head, split by the kernel that
    forms each product (C = 64):
      preparation: K K^T and Q K^T once per key head (4 C d_k / r, r = H_v/H_k),
                   W = T diag(.) K (2 C d_k), U0 = T diag(beta) V (2 C d_v)
      scan:        W S, Q S, K^T U (6 d_k d_v) and P U (2 C d_v)
    The sum is 8 C d + 6 d^2 = 163 840 at d = 128, r = 2 (the triangular
    solve is not counted)."""
    r = H_v // H_k
    prep = 4 * C * d_k // r + 2 * C * d_k + 2 * C * d_v
    scan = 2 * C * d_v + 6 * d_k * d_v
    return prep, scan


PEAK_LIB = os.path.join(ROOT, "gated_deltanet_rule_amd", "libgdnpeak.so")


def measure_peaks(dev, reps=5):
    """Measured machine peaks on this GPU (libgdnpeak.so): dense bf16 MFMA
    throughput (independent 16x16x32 products on every SIMD), and HBM
    streaming copy and read rates over 1 GiB buffers (4x the last-level
    cache).  Median of `reps` timed launches after one untimed launch."""
    import ctypes
    lib = ctypes.CDLL(PEAK_LIB)
    lib.gdn_peak_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.gdn_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                  ctypes.c_void_p]
    lib.gdn_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count

    def timed(fn):
        fn()
        out = []
        for _ in range(reps):
            t = Timer(stream, 2)
            t.mark(0)
            fn()
            t.mark(1)
            torch.cuda.synchronize()
            out.append(t.ms(0, 1))
        return statistics.median(out)

    sink = torch.zeros(1 << 16, dtype=torch.float32, device=dev)
    grid, iters = 4 * cus, 4000
    settle(lambda: lib.gdn_peak_mfma_bf16(grid, 200, ctypes.c_void_p(sink.data_ptr()), sp), ms=50)
    ms = timed(lambda: lib.gdn_peak_mfma_bf16(grid, iters, ctypes.c_void_p(sink.data_ptr()), sp))
    mfma = grid * 8 * iters * 8 * 16 * 16 * 32 * 2 / (ms * 1e-3) / 1e12
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    # the streaming rate depends on how many accesses are in flight: the best
    # of a few grid sizes (2 to 16 workgroups of 256 per CU) is the peak
    copy, read = {}, {}
    for per_cu in (2, 4, 8, 16):
        g = per_cu * cus
        ms_c = timed(lambda: lib.gdn_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                               nbytes, g, sp))
        ms_r = timed(lambda: lib.gdn_peak_read(ctypes.c_void_p(src.data_ptr()), nbytes, g,
                                               ctypes.c_void_p(sink.data_ptr()), sp))
        copy[per_cu] = 2 * nbytes / (ms_c * 1e-3) / 1e9
        read[per_cu] = nbytes / (ms_r * 1e-3) / 1e9
    assert torch.equal(dst[:1024], src[:1024])
    del src, dst
    return {"mfma_bf16_tflops": mfma, "hbm_copy_gbs": max(copy.values()),
            "hbm_read_gbs": max(read.values()),
            "hbm_copy_gbs_by_workgroups_per_cu": copy, "hbm_read_gbs_by_workgroups_per_cu": read,
            "what": "bf16 16x16x32 MFMA, 8 independent accumulators per wave, 4 x 512-thread "
                    "workgroups per CU; copy and read of 1 GiB (4x the last-level cache) with 16-byte "
                    "non-temporal accesses, best of 2-16 workgroups per CU (copy counts read + "
                    "written bytes)"}


def to_dev(case, dev):
    dt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
    f = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(t)
    return dict(q=f(case.q, dt), k=f(case.k, dt), v=f(case.v, dt), g=f(case.g),
                beta=f(case.beta), pool=f(case.pool), cu=f(case.cu_seqlens, torch.int32),
                slot_in=f(case.slot_in, torch.int32), slot_out=f(case.slot_out, torch.int32))


# Before each measurement the workload runs back to back for this long,
# untimed: the GPU's clocks take about 10 ms of sustained work to settle and
# drop again within a fraction of a second of idling (the T=4096 prefill step:
# 128 us over the first 20 steps, 112 us once settled).
SETTLE_MS = 100.0


def settle(call, ms=SETTLE_MS):
    """Run `call` back to back for at least `ms` of wall time (untimed)."""
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            call()
        torch.cuda.synchronize()


class Timer:
    """HIP events on the stream the kernels are launched on."""

    def __init__(self, stream, n):
        self.stream = stream
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    def mark(self, i):
        self.ev[i].record(self.stream)

    def ms(self, i, j):
        return self.ev[i].elapsed_time(self.ev[j])


def bench_prefill(gdn, dev, steps, warmup):
    case = gi.config1(**WG)
    d = to_dev(case, dev)
    out = torch.empty(d["v"].shape, dtype=torch.float32, device=dev)
    state_out = torch.empty_like(d["pool"])
    plan = gdn.PrefillPlan(d["q"], d["v"], out, case.n_seqs, state=state_out)
    stream = torch.cuda.current_stream()

    prep = lambda: plan.prepare(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], stream=stream)
    scan = lambda: plan.scan(d["pool"], state_out, out, d["slot_in"], d["slot_out"], stream=stream)

    def step():
        prep()
        scan()

    settle(step)
    for _ in range(warmup):
        step()
    # the step rate: steps issued back to back, nothing else on the stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / steps
    # per-kernel launch durations: each kernel launched K times back to back
    # between two HIP events on the launch stream (an event recorded between
    # two launches would add the dispatch gap after it to every interval).
    # The scans re-read the factors of the last preparation, as in a step,
    # and both kernels give the same results on every repeat.
    t = Timer(stream, 3)
    t.mark(0)
    for _ in range(steps):
        prep()
    t.mark(1)
    for _ in range(steps):
        scan()
    t.mark(2)
    torch.cuda.synchronize()
    prep_ms = t.ms(0, 1) / steps
    scan_ms = t.ms(1, 2) / steps
    assert torch.isfinite(out).all() and torch.isfinite(state_out).all()
    T, H_v = case.total_tokens, case.H_v
    fp, fs = prefill_flops_per_token_head(case.H_k, case.H_v, case.d_k, case.d_v)
    units = T * H_v
    kern = {
        # one sequence: the chunks follow from T, no chunk-table launch
        "prepare": {"kernels": "prep_kernel", "mean_ms": prep_ms,
                    "flops_per_token_head": fp,
                    "tflops": fp * units / (prep_ms * 1e-3) / 1e12},
        "scan": {"kernels": "scan_kernel", "mean_ms": scan_ms, "flops_per_token_head": fs,
                 "tflops": fs * units / (scan_ms * 1e-3) / 1e12},
    }
    dom = "scan" if scan_ms >= prep_ms else "prepare"
    ach = kern[dom]["tflops"]
    roof = {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": ach / PEAK_BF16_TFLOPS, "traffic": measured_traffic(dom),
            "traffic_unit": "bytes per launch", "kernel": kern[dom]["kernels"],
            "flops_per_token_head": kern[dom]["flops_per_token_head"],
            "units_per_launch": units,
            "flops_per_launch": kern[dom]["flops_per_token_head"] * units,
            "mean_launch_ms": kern[dom]["mean_ms"]}
    whole = (fp + fs) * units / (ms_step * 1e-3) / 1e12
    step = {"flops_per_token_head": fp + fs, "flops_per_step": (fp + fs) * units,
            "achieved": whole, "unit": "TFLOP/s", "frac": whole / PEAK_BF16_TFLOPS}
    return case, dict(ms_step=ms_step, tokens_s=T / (ms_step * 1e-3), roofline=roof,
                      kernels=kern, step=step)


def decode_bytes_per_step(dc, in_bytes=2, out_bytes=4):
    N, H_k, H_v, dk, dv = dc.n_seqs, dc.H_k, dc.H_v, dc.d_k, dc.d_v
    state = N * H_v * dk * dv * 4 * 2
    qk = N * H_k * dk * in_bytes * 2
    v = N * H_v * dv * in_bytes
    o = N * H_v * dv * out_bytes
    gb = N * H_v * 4 * 2
    return state + qk + v + o + gb + N * 4 * 2


def bench_decode(gdn, dev, reps=3):
    dc = gi.config2(**WG)
    dt = torch.bfloat16
    f = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(t)
    q, k, v = f(dc.q, dt), f(dc.k, dt), f(dc.v, dt)
    g, b = f(dc.g), f(dc.beta)
    pool = f(dc.pool)
    pool2 = pool.clone()
    slots = f(dc.slots, torch.int32)
    outs = torch.empty(v.shape, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    S = dc.n_steps
    res = {}
    settle(lambda: gdn.decode_step(q[0], k[0], v[0], g[0], b[0], pool2, pool2, outs[0], slots, slots,
                                   stream=stream))
    for mode in ("in_place", "ping_pong"):
        per_rep = []
        for rep in range(reps + 1):
            t = Timer(stream, 2)
            torch.cuda.synchronize()
            t.mark(0)
            for s in range(S):
                if mode == "in_place":
                    src, dst = pool, pool
                else:
                    src, dst = (pool, pool2) if s % 2 == 0 else (pool2, pool)
                gdn.decode_step(q[s], k[s], v[s], g[s], b[s], src, dst, outs[s], slots, slots,
                                stream=stream)
            t.mark(1)
            torch.cuda.synchronize()
            if rep == 0:
                continue  # warm-up pass
            per_rep.append(t.ms(0, 1))
        # the 128 launches run back to back between one pair of events
        ms_128 = statistics.median(per_rep)
        launch_ms = ms_128 / S
        by = decode_bytes_per_step(dc)
        gbs = by / (launch_ms * 1e-3) / 1e9
        res[mode] = {"ms_per_128_steps": ms_128, "mean_launch_ms": launch_ms,
                     "tokens_s": dc.n_seqs * S / (ms_128 * 1e-3),
                     "bytes_per_launch": by, "achieved_gbs": gbs,
                     "frac": gbs / PEAK_HBM_GBS}
    assert torch.isfinite(outs).all()
    # context for the HBM fraction: a plain device copy (PyTorch's own copy
    # kernel) of the pool, i.e. the same bytes read once and written once
    copy_ms = []
    for rep in range(21):
        t = Timer(stream, 2)
        t.mark(0)
        pool2.copy_(pool)
        t.mark(1)
        torch.cuda.synchronize()
        if rep:
            copy_ms.append(t.ms(0, 1))
    cms = statistics.median(copy_ms)
    cby = 2 * pool.numel() * pool.element_size()
    res["copy_reference"] = {"what": "torch copy_ of the 128 MiB pool into a second pool",
                             "bytes": cby, "ms": cms, "achieved_gbs": cby / (cms * 1e-3) / 1e9,
                             "frac": cby / (cms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    ip, pp = res["in_place"], res["ping_pong"]
    # the headline rate is the ping-pong run: its two pools (256 MiB) do not
    # fit the 256 MB last-level cache, so its bytes come from HBM; the in-place
    # pool (128 MiB) can be served partly from that cache
    return {"workload": "decode: 64 sequences x 128 steps, H_k=16 H_v=32 d=128, bf16 in, "
                        "fp32 out, fp32 state slots (two 128 MiB pools, ping-pong)",
            "value": pp["tokens_s"], "unit": "tokens/s",
            "ms_per_step": pp["mean_launch_ms"],
            "roofline": {"bound": "hbm", "achieved": pp["achieved_gbs"], "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": pp["frac"], "traffic": measured_traffic("decode"),
                         "traffic_unit": "bytes per launch (in-place run)",
                         "kernel": "decode_kernel", "bytes_per_launch": pp["bytes_per_launch"],
                         "mean_launch_ms": pp["mean_launch_ms"]},
            "ping_pong": pp, "in_place": ip, "copy_reference": res["copy_reference"]}


def bench_decode_multi(gdn, dev, tokens=4, reps=200):
    """gdn_recurrent_multi: 64 sequences x `tokens` tokens (speculative
    verification), state pool in place; HBM roofline on state + I/O bytes."""
    case = gi.make_case(f"spec64x{tokens}", [tokens] * 64, dtype="bf16", seed=40 + tokens,
                        final_gates=workload_gates, **gi.QWEN3_NEXT_HEADS)
    d = to_dev(case, dev)
    out = torch.empty(d["v"].shape, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    call = lambda: gdn.decode_multi(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"],
                                    d["pool"], out, d["cu"], d["slot_in"], d["slot_out"],
                                    stream=stream)
    settle(call)
    t = Timer(stream, 2)
    torch.cuda.synchronize()
    t.mark(0)
    for r in range(reps):
        call()
    t.mark(1)
    torch.cuda.synchronize()
    ms = t.ms(0, 1) / reps
    N, H_k, H_v, dk, dv, T = 64, case.H_k, case.H_v, case.d_k, case.d_v, case.total_tokens
    by = N * H_v * dk * dv * 4 * 2 + T * (2 * H_k * dk * 2 + H_v * dv * 2 + H_v * dv * 4 + H_v * 8)
    gbs = by / (ms * 1e-3) / 1e9
    return {"workload": f"multi-token decode: 64 sequences x {tokens} tokens, H_k=16 H_v=32 "
                        "d=128, bf16 in, fp32 out, state slots in place",
            "ms_per_call": ms, "tokens_s": T / (ms * 1e-3),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS, "kernel": "decode_multi_kernel",
                         "bytes_per_launch": by}}


def _layer_dev(case, L, dev):
    dt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
    f = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(t)
    n = case.pool.shape[0]
    rows = np.concatenate([L.conv_pool.reshape(n, -1), case.pool.reshape(n, -1)], axis=1)
    return dict(qkv=f(L.qkv, dt), a=f(case.raw_a), b=f(case.raw_b), ssm_a=f(case.ssm_a),
                ssm_dt=f(case.ssm_dt), rows=f(rows), conv_w=f(L.conv_w), z=f(L.z, dt),
                norm_w=f(L.norm_w), cu=f(case.cu_seqlens, torch.int32),
                slot_in=f(case.slot_in, torch.int32), slot_out=f(case.slot_out, torch.int32))


def bench_layer_prefill(gdn, dev, reps=50):
    """The fused layer path on the T=4096 prefill: mixed q|k|v rows through
    the convolution prologue, raw gate projections, gated RMSNorm epilogue,
    bf16 output; one gdn_chunked_prefill call per step."""
    case = gi.config1(**WG)
    L = gi.make_layer_inputs(case.total_tokens, case.pool.shape[0], case.H_k, case.H_v, case.d_k,
                             case.d_v, "bf16", 1)
    d = _layer_dev(case, L, dev)
    out = torch.empty((case.total_tokens, case.H_v, case.d_v), dtype=torch.bfloat16, device=dev)
    rows_out = torch.empty_like(d["rows"])
    stream = torch.cuda.current_stream()
    cv = (d["conv_w"], case.H_k, case.d_k)
    dims = gdn._dims_from(d["qkv"], None, out, 0.0, 1e-6, rows_out, (d["ssm_a"], d["ssm_dt"]), cv,
                          d["z"], d["norm_w"])
    ws = torch.empty(gdn.workspace_size(dims, 1, case.total_tokens), dtype=torch.uint8, device=dev)
    call = lambda: gdn.prefill(d["qkv"], None, None, d["a"], d["b"], d["rows"], rows_out, out, d["cu"],
                               d["slot_in"], d["slot_out"], ws, stream=stream,
                               gates=(d["ssm_a"], d["ssm_dt"]), conv=cv, z=d["z"], norm_w=d["norm_w"])
    settle(call)
    t = Timer(stream, 2)
    torch.cuda.synchronize()
    t.mark(0)
    for r in range(reps):
        call()
    t.mark(1)
    torch.cuda.synchronize()
    ms = t.ms(0, 1) / reps
    assert torch.isfinite(out.float()).all()
    T = case.total_tokens
    return {"workload": "fused layer prefill: 1 x 4096 tokens, mixed bf16 q|k|v rows -> conv(4) + "
                        "SiLU, raw gates, gated RMSNorm, bf16 out, Qwen3-Next heads",
            "ms_per_call": ms, "tokens_s": T / (ms * 1e-3),
            "operands": "two-term bf16 (hi + lo) q, k, v and W: the prologue's output is not rounded "
                        "to bf16 once"}


def bench_layer_decode(gdn, dev, reps=3):
    """The fused layer path on the decode workload: 64 sequences x 128
    steps, one gdn_recurrent_step per step with the prologue (mixed rows,
    convolution state in the slot rows), raw gates and the epilogue."""
    dc = gi.config2(**WG)
    S, N = dc.n_steps, dc.n_seqs
    L = gi.make_layer_inputs(S * N, N, dc.H_k, dc.H_v, dc.d_k, dc.d_v, "bf16", 2)
    f = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(t)
    C = L.qkv.shape[1]
    qkv = f(L.qkv.reshape(S, N, C), torch.bfloat16)
    z = f(L.z.reshape(S, N, dc.H_v, dc.d_v), torch.bfloat16)
    rows = f(np.concatenate([L.conv_pool.reshape(N, -1), dc.pool.reshape(N, -1)], axis=1))
    a, b = f(dc.raw_a), f(dc.raw_b)
    gates = (f(dc.ssm_a), f(dc.ssm_dt))
    cv = (f(L.conv_w), dc.H_k, dc.d_k)
    nw = f(L.norm_w)
    slots = f(dc.slots, torch.int32)
    outs = torch.empty((S, N, dc.H_v, dc.d_v), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    rows2 = rows.clone()
    settle(lambda: gdn.decode_step(qkv[0], None, None, a[0], b[0], rows2, rows2, outs[0], slots, slots,
                                   stream=stream, gates=gates, conv=cv, z=z[0], norm_w=nw))
    del rows2
    per = []
    for rep in range(reps + 1):
        t = Timer(stream, 2)
        torch.cuda.synchronize()
        t.mark(0)
        for s in range(S):
            gdn.decode_step(qkv[s], None, None, a[s], b[s], rows, rows, outs[s], slots, slots,
                            stream=stream, gates=gates, conv=cv, z=z[s], norm_w=nw)
        t.mark(1)
        torch.cuda.synchronize()
        if rep:
            per.append(t.ms(0, 1))
    ms = statistics.median(per)
    assert torch.isfinite(outs.float()).all()
    conv_state = N * C * 3 * 4 * 2
    # state, mixed rows (the q|k|v bytes of the plain step), bf16 out, z, and
    # the convolution state read and written
    by = decode_bytes_per_step(dc, out_bytes=2) + N * dc.H_v * dc.d_v * 2 + conv_state
    gbs = by / (ms / S * 1e-3) / 1e9
    return {"workload": "fused layer decode: 64 sequences x 128 steps, mixed bf16 rows -> conv(4) "
                        "+ SiLU, raw gates, gated RMSNorm, bf16 out, state + conv state in slot rows",
            "ms_per_step": ms / S, "tokens_s": N * S / (ms * 1e-3),
            "bytes_per_step": by, "achieved_gbs": gbs, "frac": gbs / PEAK_HBM_GBS,
            "kernels": "decode_kernel (prologue, epilogue and the convolution state update in one "
                       "launch: one workgroup per (sequence, key head))"}


def bench_layer_multi(gdn, dev, tokens=4, reps=200):
    """The fused layer path on the multi-token decode workload: 64 sequences x
    `tokens` tokens in one gdn_recurrent_multi call with the prologue (mixed
    rows, convolution state in the slot rows), raw gates and the epilogue,
    bf16 out, slot rows in place."""
    case = gi.make_case(f"layer_spec64x{tokens}", [tokens] * 64, dtype="bf16", seed=40 + tokens,
                        final_gates=workload_gates, **gi.QWEN3_NEXT_HEADS)
    L = gi.make_layer_inputs(case.total_tokens, case.pool.shape[0], case.H_k, case.H_v, case.d_k,
                             case.d_v, "bf16", 40 + tokens)
    d = _layer_dev(case, L, dev)
    out = torch.empty((case.total_tokens, case.H_v, case.d_v), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    cv = (d["conv_w"], case.H_k, case.d_k)
    call = lambda: gdn.decode_multi(d["qkv"], None, None, d["a"], d["b"], d["rows"], d["rows"], out,
                                    d["cu"], d["slot_in"], d["slot_out"], stream=stream,
                                    gates=(d["ssm_a"], d["ssm_dt"]), conv=cv, z=d["z"],
                                    norm_w=d["norm_w"])
    settle(call)
    t = Timer(stream, 2)
    torch.cuda.synchronize()
    t.mark(0)
    for r in range(reps):
        call()
    t.mark(1)
    torch.cuda.synchronize()
    ms = t.ms(0, 1) / reps
    assert torch.isfinite(out.float()).all()
    N, H_k, H_v, dk, dv, T = 64, case.H_k, case.H_v, case.d_k, case.d_v, case.total_tokens
    conv_dim = 2 * H_k * dk + H_v * dv
    # state and convolution state read and written; per token the mixed rows,
    # z, the bf16 output and the raw gate projections
    by = N * (H_v * dk * dv * 4 + conv_dim * 3 * 4) * 2 + T * (conv_dim * 2 + H_v * dv * 2 * 2 + H_v * 8)
    gbs = by / (ms * 1e-3) / 1e9
    return {"workload": f"fused layer multi-token decode: 64 sequences x {tokens} tokens, mixed bf16 rows "
                        "-> conv(4) + SiLU, raw gates, gated RMSNorm, bf16 out, state + conv state in "
                        "slot rows",
            "ms_per_call": ms, "tokens_s": T / (ms * 1e-3), "bytes_per_call": by, "achieved_gbs": gbs,
            "frac": gbs / PEAK_HBM_GBS, "kernels": "decode_multi_kernel (one launch per call)"}


def bench_varlen(gdn, dev, reps=20):
    """The varlen batch as one gdn_chunked_prefill call (it runs as chunk
    ranges of about 64 chunks), and as the two split-phase calls (one range
    over the whole batch) for comparison."""
    case = gi.config3(**WG)
    d = to_dev(case, dev)
    out = torch.empty(d["v"].shape, dtype=torch.float32, device=dev)
    pool_out = d["pool"].clone()
    stream = torch.cuda.current_stream()
    dims = gdn._dims_from(d["q"], d["v"], out, 0.0, 1e-6, pool_out)
    ws = torch.empty(gdn.workspace_size(dims, case.n_seqs, case.total_tokens), dtype=torch.uint8,
                     device=dev)
    call = lambda: gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], pool_out, out,
                               d["cu"], d["slot_in"], d["slot_out"], ws, stream=stream)
    plan = gdn.PrefillPlan(d["q"], d["v"], out, case.n_seqs, state=pool_out, workspace=ws)
    split = lambda: (plan.prepare(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], stream=stream),
                     plan.scan(d["pool"], pool_out, out, d["slot_in"], d["slot_out"], stream=stream))
    res = {}
    for name, fn in (("call", call), ("split", split)):
        settle(fn)
        t = Timer(stream, 2)
        torch.cuda.synchronize()
        t.mark(0)
        for _ in range(reps):
            fn()
        t.mark(1)
        torch.cuda.synchronize()
        res[name] = t.ms(0, 1) / reps
    total = res["call"]
    T = case.total_tokens
    fp, fs = prefill_flops_per_token_head(case.H_k, case.H_v, case.d_k, case.d_v)
    tf = (fp + fs) * T * case.H_v / (total * 1e-3) / 1e12
    return {"workload": "varlen: 8 sequences {17,64,65,300,512,1023,2048,8192} = 12221 tokens, "
                        "scattered slots", "ms_per_call": total,
            "split_phase_ms": res["split"], "tokens_s": T / (total * 1e-3), "tflops": tf,
            "mfma_frac": tf / PEAK_BF16_TFLOPS}


def bench_stream(gdn, dev, reps=2):
    case = gi.config4(**WG)
    d = to_dev(case, dev)
    T, U = case.total_tokens, 512
    out = torch.empty(d["v"].shape, dtype=torch.float32, device=dev)
    pool = d["pool"].clone()
    plan = gdn.PrefillPlan(d["q"][:U], d["v"][:U], out[:U], 1, state=pool)
    cu = torch.tensor([0, U], dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def run():
        for s in range(0, T, U):
            sl_in = d["slot_in"] if s == 0 else d["slot_out"]
            plan.prepare(d["q"][s:s + U], d["k"][s:s + U], d["v"][s:s + U], d["g"][s:s + U],
                         d["beta"][s:s + U], cu, stream=stream)
            plan.scan(pool, pool, out[s:s + U], sl_in, d["slot_out"], stream=stream)

    settle(run)
    times = []
    for _ in range(reps):
        pool.copy_(d["pool"])
        t = Timer(stream, 2)
        torch.cuda.synchronize()
        t.mark(0)
        run()
        t.mark(1)
        torch.cuda.synchronize()
        times.append(t.ms(0, 1))
    ms = statistics.median(times)
    eager_out, eager_pool = out.clone(), pool.clone()
    # the same 256 launches captured once into a HIP graph and replayed: the
    # host's launch gaps between the short kernels drop out
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        pool.copy_(d["pool"])
        run()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gstream = torch.cuda.current_stream()
        for s0 in range(0, T, U):
            sl_in = d["slot_in"] if s0 == 0 else d["slot_out"]
            plan.prepare(d["q"][s0:s0 + U], d["k"][s0:s0 + U], d["v"][s0:s0 + U], d["g"][s0:s0 + U],
                         d["beta"][s0:s0 + U], cu, stream=gstream)
            plan.scan(pool, pool, out[s0:s0 + U], sl_in, d["slot_out"], stream=gstream)
    gtimes = []
    for _ in range(reps + 1):
        pool.copy_(d["pool"])
        t = Timer(stream, 2)
        torch.cuda.synchronize()
        t.mark(0)
        graph.replay()
        t.mark(1)
        torch.cuda.synchronize()
        gtimes.append(t.ms(0, 1))
    assert torch.equal(out, eager_out) and torch.equal(pool, eager_pool), "graph replay differs from eager"
    gms = statistics.median(gtimes[1:])
    # the same 65536 tokens as one gdn_chunked_prefill call (chunk ranges of
    # 64 chunks, one range of factor slots in the workspace)
    cu1 = torch.tensor([0, T], dtype=torch.int32, device=dev)
    dims = gdn._dims_from(d["q"], d["v"], out, 0.0, 1e-6, pool)
    ws1 = torch.empty(gdn.chunked_workspace_size(dims, 1, T), dtype=torch.uint8, device=dev)
    one = lambda: gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], pool, out, cu1,
                              d["slot_in"], d["slot_out"], ws1, stream=stream)
    settle(one)
    t = Timer(stream, 2)
    torch.cuda.synchronize()
    t.mark(0)
    for _ in range(reps + 1):
        one()
    t.mark(1)
    torch.cuda.synchronize()
    oms = t.ms(0, 1) / (reps + 1)
    fp, fs = prefill_flops_per_token_head(case.H_k, case.H_v, case.d_k, case.d_v)
    tf = (fp + fs) * T * case.H_v / (ms * 1e-3) / 1e12
    return {"workload": "stream: 65536 tokens as 128 calls of 512, state carried in place",
            "ms_total": ms, "us_per_call": ms * 1e3 / (T // U), "tokens_s": T / (ms * 1e-3),
            "tflops": tf, "mfma_frac": tf / PEAK_BF16_TFLOPS,
            "hip_graph": {"ms_total": gms, "us_per_call": gms * 1e3 / (T // U),
                          "tokens_s": T / (gms * 1e-3)},
            "one_call": {"ms": oms, "tokens_s": T / (oms * 1e-3),
                         "workspace_bytes": ws1.numel()}}


def cpu_baseline(case, min_s=10.0, max_reps=40):
    """The oracle on the whole prefill workload, repeated until about
    min_s seconds of wall time (at least 3 runs); median per run."""
    import oracle
    threads = oracle.default_threads()
    walls = []
    t_start = time.perf_counter()
    while len(walls) < 3 or (time.perf_counter() - t_start < min_s and len(walls) < max_reps):
        t0 = time.perf_counter()
        oracle.run_case(case, threads=threads)
        walls.append(time.perf_counter() - t0)
    reps = len(walls)
    w = statistics.median(walls)
    return {"value": case.total_tokens / w, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the whole prefill workload (1 x {case.total_tokens} tokens, all "
                      f"{case.H_v} value heads), fp64 sequential recurrence threaded over heads, "
                      f"median of {reps} runs ({w:.2f} s wall each)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="headline prefill + decode only")
    ap.add_argument("--decode-only", action="store_true",
                    help="the decode workload only (for hardware-counter runs)")
    ap.add_argument("--layer-only", action="store_true",
                    help="the fused layer prefill and decode only (for kernel traces)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="headline prefill only (for hardware-counter runs)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run 3 plain device copies of this many MiB (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} (WORLD_SIZE {world}) is not "
              "supported: the operator is benchmarked on a single MI355X", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import gated_deltanet_rule_amd as gdn
    dev = torch.device("cuda:0")

    if args.layer_only:
        log("fused layer prefill T=4096 ...")
        lp = bench_layer_prefill(gdn, dev)
        log("fused layer decode 64x128 ...")
        ld = bench_layer_decode(gdn, dev)
        log("fused layer multi-token decode 64x4 ...")
        lm = bench_layer_multi(gdn, dev)
        log(f"  {lp['ms_per_call']*1e3:.1f} us/call, {ld['ms_per_step']*1e3:.1f} us/step, "
            f"{lm['ms_per_call']*1e3:.1f} us/multi call")
        return
    if args.copy_mib:
        n = args.copy_mib << 18
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration: 3 copies of {args.copy_mib} MiB")
        del src, dst
    if args.decode_only:
        log("decode 64x128 ...")
        dec = bench_decode(gdn, dev, reps=1)
        log(f"  {dec['ms_per_step']*1e3:.2f} us/step, {dec['roofline']['achieved']:.0f} GB/s "
            f"(device copy of the pool: {dec['copy_reference']['achieved_gbs']:.0f} GB/s)")
        return
    log("prefill T=4096 ...")
    case, pf = bench_prefill(gdn, dev, args.steps, args.warmup)
    log(f"  {pf['ms_step']:.4f} ms/step, {pf['tokens_s']:.4g} tok/s")
    if args.prefill_only:
        return
    log("measured peaks ...")
    peaks = measure_peaks(dev)
    log(f"  bf16 MFMA {peaks['mfma_bf16_tflops']:.0f} TFLOP/s, HBM copy {peaks['hbm_copy_gbs']:.0f} GB/s, "
        f"read {peaks['hbm_read_gbs']:.0f} GB/s")
    for r in (pf["roofline"], pf["step"]):
        r["peak_measured"] = peaks["mfma_bf16_tflops"]
        r["frac_measured"] = r["achieved"] / peaks["mfma_bf16_tflops"]
    log("decode 64x128 ...")
    dec = bench_decode(gdn, dev)
    dec["roofline"]["peak_measured"] = peaks["hbm_copy_gbs"]
    dec["roofline"]["frac_measured"] = dec["roofline"]["achieved"] / peaks["hbm_copy_gbs"]
    log(f"  {dec['ms_per_step']*1e3:.2f} us/step, {dec['roofline']['achieved']:.0f} GB/s "
        f"(device copy of the pool: {dec['copy_reference']['achieved_gbs']:.0f} GB/s)")
    extra = {}
    log("multi-token decode 64x4 ...")
    extra["decode_multi"] = bench_decode_multi(gdn, dev)
    log(f"  {extra['decode_multi']['ms_per_call']*1e3:.1f} us/call, "
        f"{extra['decode_multi']['roofline']['achieved']:.0f} GB/s")
    if not args.quick:
        log("fused layer prefill T=4096 ...")
        extra["layer_prefill"] = bench_layer_prefill(gdn, dev)
        log(f"  {extra['layer_prefill']['ms_per_call']*1e3:.1f} us/call")
        log("fused layer decode 64x128 ...")
        extra["layer_decode"] = bench_layer_decode(gdn, dev)
        log(f"  {extra['layer_decode']['ms_per_step']*1e3:.1f} us/step")
        log("fused layer multi-token decode 64x4 ...")
        extra["layer_multi"] = bench_layer_multi(gdn, dev)
        log(f"  {extra['layer_multi']['ms_per_call']*1e3:.1f} us/call")
        log("varlen ...")
        extra["varlen"] = bench_varlen(gdn, dev)
        log(f"  {extra['varlen']['ms_per_call']*1e3:.0f} us/call "
            f"({extra['varlen']['split_phase_ms']*1e3:.0f} us as split-phase calls)")
        log("stream 65536 ...")
        extra["stream"] = bench_stream(gdn, dev)
        log(f"  {extra['stream']['us_per_call']:.1f} us/call, "
            f"{extra['stream']['hip_graph']['us_per_call']:.1f} us/call replayed from a HIP graph; "
            f"as one call {extra['stream']['one_call']['ms']:.2f} ms")
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(case)

    line = {
        "metric": METRIC,
        "value": pf["tokens_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pf["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill: 1 sequence x 4096 tokens, H_k=16 H_v=32 d_k=d_v=128, "
                               "chunk 64, bf16 q/k/v, fp32 g/beta/state, fp32 out",
                   "tokens": case.total_tokens, "H_k": 16, "H_v": 32, "d_k": 128, "d_v": 128,
                   "chunk": C, "parallelism": "single GPU"},
        "roofline": pf["roofline"],
        "prefill_kernels": pf["kernels"],
        "prefill_step_roofline": pf["step"],
        "measured_peaks": peaks,
        "decode": dec,
        "cpu_baseline": cpu,
    }
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
