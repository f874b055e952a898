"""Helpers for the GPU parity tests: move a seeded workload to the device, run
it through libgdn's C ABI (via the thin binding), and compare with the fp64
oracle under the tolerance the operator is held to:

    max |gpu - oracle| <= tol * rms(oracle)   for outputs and final states,
    tol = 1e-4 (fp32 q/k/v) or 2e-2 (bf16 q/k/v).

With a bf16 output the result is additionally rounded once to bf16 (round to
nearest even: relative error <= 2^-8), so each output element is held to
    |gpu - oracle| <= tol * rms(oracle) + 2^-8 * |oracle|.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import torch

import workloads as gi
import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tdt(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def dev_case(case, device="cuda"):
    dt = tdt(case.dtype)
    f = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(device).to(t)
    return dict(
        q=f(case.q, dt), k=f(case.k, dt), v=f(case.v, dt), g=f(case.g), beta=f(case.beta),
        pool=f(case.pool), cu=f(case.cu_seqlens, torch.int32),
        slot_in=f(case.slot_in, torch.int32), slot_out=f(case.slot_out, torch.int32),
        raw_a=f(case.raw_a), raw_b=f(case.raw_b), ssm_a=f(case.ssm_a), ssm_dt=f(case.ssm_dt))


def _gate_args(d, raw_gates):
    """(g, beta, gates) for the binding: the final gates, or the raw
    projections plus (ssm_a, ssm_dt) for the in-kernel activations."""
    if raw_gates:
        return d["raw_a"], d["raw_b"], (d["ssm_a"], d["ssm_dt"])
    return d["g"], d["beta"], None


def gpu_prefill(case, d=None, inplace=True, chunks=None, out_dtype=torch.float32,
                raw_gates=False):
    """Run a Case through gdn.prefill.  `chunks`: split a single-sequence case
    into consecutive calls of that many tokens (state carried in place)."""
    import gated_deltanet_rule_amd as gdn
    d = d or dev_case(case)
    T = case.total_tokens
    out = torch.empty(d["v"].shape, dtype=out_dtype, device=d["v"].device)
    pool_out = d["pool"] if inplace else torch.full_like(d["pool"], float("nan"))
    if not inplace:
        # slots that are not written must keep whatever the output pool held
        pool_out.copy_(d["pool"])
    g, beta, gates = _gate_args(d, raw_gates)
    if chunks is None:
        gdn.prefill(d["q"], d["k"], d["v"], g, beta, d["pool"], pool_out, out,
                    d["cu"], d["slot_in"], d["slot_out"], gates=gates)
    else:
        assert case.n_seqs == 1 and inplace
        for s in range(0, T, chunks):
            e = min(T, s + chunks)
            cu = torch.tensor([0, e - s], dtype=torch.int32, device=d["q"].device)
            sl_in = d["slot_in"] if s == 0 else d["slot_out"]
            gdn.prefill(d["q"][s:e], d["k"][s:e], d["v"][s:e], g[s:e], beta[s:e],
                        d["pool"], d["pool"], out[s:e], cu, sl_in, d["slot_out"], gates=gates)
    torch.cuda.synchronize()
    return out, pool_out


def gpu_decode_multi(case, d=None, inplace=True, out_dtype=torch.float32, raw_gates=False):
    """Run a Case (tokens packed by cu_seqlens) through gdn.decode_multi."""
    import gated_deltanet_rule_amd as gdn
    d = d or dev_case(case)
    out = torch.empty(d["v"].shape, dtype=out_dtype, device=d["v"].device)
    pool_out = d["pool"] if inplace else d["pool"].clone()
    g, beta, gates = _gate_args(d, raw_gates)
    gdn.decode_multi(d["q"], d["k"], d["v"], g, beta, d["pool"], pool_out, out,
                     d["cu"], d["slot_in"], d["slot_out"], gates=gates)
    torch.cuda.synchronize()
    return out, pool_out


def oracle_case(case, heads=None, raw_gates=False):
    return oracle.run_case(case, heads=heads, raw_gates=raw_gates)


def rel_err(gpu, ref, bf16_out=False):
    """max |gpu - ref| / rms(ref); with bf16_out the allowance 2^-8 |ref| for
    the final rounding is subtracted first."""
    ref = np.asarray(ref, np.float64)
    gpu = np.asarray(gpu, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    d = np.abs(gpu - ref)
    if bf16_out:
        d = np.maximum(d - 2.0 ** -8 * np.abs(ref), 0.0)
    # a reference below fp32's useful range (e.g. a state decayed by e^-400)
    # is compared in absolute terms against 1e-30
    return float(np.max(d)) / max(rms, 1e-30), rms


def compare_prefill(case, out, pool_out, ref_out, ref_state, heads=None, tol=None):
    """Returns (out_err, state_err) relative to rms; asserts finiteness."""
    tol = tol or TOL[case.dtype]
    hs = list(range(case.H_v)) if heads is None else list(heads)
    assert bool(torch.isfinite(out.float()).all()), "non-finite output"
    o = out[:, hs].float().cpu().numpy().astype(np.float64)
    eo, _ = rel_err(o, ref_out[:, hs], bf16_out=out.dtype == torch.bfloat16)
    st = np.stack([pool_out[int(case.slot_out[i])].cpu().numpy().astype(np.float64)
                   for i in range(case.n_seqs)])
    es, _ = rel_err(st[:, hs], ref_state[:, hs])
    say(f"  {case.name}: out err/rms = {eo:.3e}, state err/rms = {es:.3e} (tol {tol:g})")
    assert eo <= tol, f"output error {eo:.3e} > {tol}"
    assert es <= tol, f"state error {es:.3e} > {tol}"
    return eo, es


def run_decode(dc, device="cuda", inplace=True, out_dtype=torch.float32, raw_gates=False):
    """Run a DecodeCase step by step; returns (outs [steps, N, H_v, d_v], pool)."""
    import gated_deltanet_rule_amd as gdn
    dt = tdt(dc.dtype)
    f = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(device).to(t)
    q, k, v = f(dc.q, dt), f(dc.k, dt), f(dc.v, dt)
    g, b = (f(dc.raw_a), f(dc.raw_b)) if raw_gates else (f(dc.g), f(dc.beta))
    gates = (f(dc.ssm_a), f(dc.ssm_dt)) if raw_gates else None
    pool = f(dc.pool)
    slots = f(dc.slots, torch.int32)
    outs = torch.empty(v.shape, dtype=out_dtype, device=device)
    pool_b = pool if inplace else pool.clone()
    for s in range(dc.n_steps):
        src, dst = (pool, pool) if inplace else ((pool, pool_b) if s % 2 == 0 else (pool_b, pool))
        gdn.decode_step(q[s], k[s], v[s], g[s], b[s], src, dst, outs[s], slots, slots,
                        gates=gates)
    torch.cuda.synchronize()
    final = pool if (inplace or dc.n_steps % 2 == 0) else pool_b
    return outs, final


def oracle_decode(dc, heads=None, raw_gates=False):
    if raw_gates:
        g, b = oracle.gates(dc.raw_a.reshape(-1, dc.H_v), dc.raw_b.reshape(-1, dc.H_v),
                            dc.ssm_a, dc.ssm_dt)
        shape = (dc.n_steps, dc.n_seqs, dc.H_v)
        dc = dataclasses.replace(dc, g=g.reshape(shape), beta=b.reshape(shape))
    q, k, v, g, b, cu = gi.decode_as_sequences(dc)
    s0 = np.stack([dc.pool[dc.slots[i]] for i in range(dc.n_seqs)]).astype(np.float64)
    out, sf = oracle.run(q, k, v, g, b, cu, s0, heads=heads)
    # back to [steps, N, ...]
    out = out.reshape(dc.n_seqs, dc.n_steps, dc.H_v, dc.d_v).swapaxes(0, 1)
    return out, sf


def compare_decode(dc, outs, pool, ref_out, ref_state, heads=None):
    tol = TOL[dc.dtype]
    o = outs.float().cpu().numpy().astype(np.float64)
    P = pool.cpu().numpy().astype(np.float64)
    hs = list(range(dc.H_v)) if heads is None else list(heads)
    assert np.all(np.isfinite(o))
    eo, _ = rel_err(o[:, :, hs], ref_out[:, :, hs], bf16_out=outs.dtype == torch.bfloat16)
    st = np.stack([P[dc.slots[i]] for i in range(dc.n_seqs)])
    es, _ = rel_err(st[:, hs], ref_state[:, hs])
    say(f"  {dc.name}: out err/rms = {eo:.3e}, state err/rms = {es:.3e} (tol {tol:g})")
    assert eo <= tol and es <= tol
    return eo, es


# ---------------------------------------------------------------------------
# Layer fusion: convolution prologue (mixed rows + per-slot convolution state
# at the start of each slot row) and gated RMSNorm epilogue.
# ---------------------------------------------------------------------------

def layer_pool(case, L):
    """Slot rows [n_slots, 3*conv_dim + H_v*d_k*d_v]: convolution state, then state."""
    n = case.pool.shape[0]
    return np.concatenate([L.conv_pool.reshape(n, -1), case.pool.reshape(n, -1)], axis=1)


def split_pool(case, L, rows):
    """Device slot rows -> (conv states [n, conv_dim, 3], states [n, H_v, d_k, d_v])."""
    R = rows.cpu().numpy()
    n = R.shape[0]
    c = L.conv_pool[0].size
    return R[:, :c].reshape(L.conv_pool.shape), R[:, c:].reshape(case.pool.shape)


def dev_layer(case, L, conv=True, norm=True, device="cuda"):
    """Device tensors of a layer workload: the case's q/k/v (or the mixed rows),
    gates, slot rows (or the plain pool), taps, z, norm weight."""
    import gated_deltanet_rule_amd as gdn
    d = dev_case(case, device)
    dt = tdt(case.dtype)
    f = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(device).to(t)
    d["conv_w"] = f(L.conv_w)
    d["qkv"] = f(L.qkv, dt)
    d["z"] = f(L.z, dt) if norm else None
    d["norm_w"] = f(L.norm_w) if norm else None
    if conv:
        d["pool"] = f(layer_pool(case, L))
    return d


def gpu_layer_prefill(case, L, conv=True, norm=True, raw_gates=False, out_dtype=torch.float32,
                      inplace=True, chunks=None, d=None):
    """Run a layer workload through gdn.prefill; `chunks` splits a single
    sequence into consecutive calls (state rows carried in place)."""
    import gated_deltanet_rule_amd as gdn
    d = d or dev_layer(case, L, conv, norm)
    T = case.total_tokens
    out = torch.empty((T, case.H_v, case.d_v), dtype=out_dtype, device=d["q"].device)
    pool_out = d["pool"] if inplace else d["pool"].clone()
    g, beta, gates = _gate_args(d, raw_gates)
    cv = (d["conv_w"], case.H_k, case.d_k) if conv else None

    def call(s, e, cu, sl_in):
        if conv:
            q, k, v = d["qkv"][s:e], None, None
        else:
            q, k, v = d["q"][s:e], d["k"][s:e], d["v"][s:e]
        z = d["z"][s:e] if norm else None
        gdn.prefill(q, k, v, g[s:e], beta[s:e], d["pool"], pool_out, out[s:e], cu, sl_in,
                    d["slot_out"], gates=gates, conv=cv, z=z, norm_w=d["norm_w"])

    if chunks is None:
        call(0, T, d["cu"], d["slot_in"])
    else:
        assert case.n_seqs == 1 and inplace
        for s in range(0, T, chunks):
            e = min(T, s + chunks)
            cu = torch.tensor([0, e - s], dtype=torch.int32, device=d["q"].device)
            call(s, e, cu, d["slot_in"] if s == 0 else d["slot_out"])
    torch.cuda.synchronize()
    return out, pool_out


def gpu_layer_multi(case, L, conv=True, norm=True, raw_gates=False, out_dtype=torch.float32,
                    inplace=True):
    import gated_deltanet_rule_amd as gdn
    d = dev_layer(case, L, conv, norm)
    T = case.total_tokens
    out = torch.empty((T, case.H_v, case.d_v), dtype=out_dtype, device=d["q"].device)
    pool_out = d["pool"] if inplace else d["pool"].clone()
    g, beta, gates = _gate_args(d, raw_gates)
    q, k, v = (d["qkv"], None, None) if conv else (d["q"], d["k"], d["v"])
    gdn.decode_multi(q, k, v, g, beta, d["pool"], pool_out, out, d["cu"], d["slot_in"],
                     d["slot_out"], gates=gates,
                     conv=(d["conv_w"], case.H_k, case.d_k) if conv else None,
                     z=d["z"], norm_w=d["norm_w"])
    torch.cuda.synchronize()
    return out, pool_out


def oracle_layer(case, L, conv=True, norm=True, raw_gates=False, heads=None):
    """fp64 oracle of the layer workload: (out, states, conv states) per sequence."""
    from oracle import layer as OL
    N = case.n_seqs
    s0 = np.zeros((N, case.H_v, case.d_k, case.d_v))
    c0 = np.zeros((N,) + L.conv_pool.shape[1:])
    for i in range(N):
        if case.slot_in[i] >= 0:
            s0[i] = case.pool[case.slot_in[i]]
            c0[i] = L.conv_pool[case.slot_in[i]]
    g, beta = case.g, case.beta
    if raw_gates:
        g, beta = oracle.gates(case.raw_a, case.raw_b, case.ssm_a, case.ssm_dt)
    z = L.z if norm else None
    if conv:
        return OL.run_layer(case.H_k, case.H_v, case.d_k, case.d_v, L.qkv, L.conv_w, c0, g, beta,
                            case.cu_seqlens, s0, z, L.norm_w, heads=heads)
    out, sf = oracle.run(case.q, case.k, case.v, g, beta, case.cu_seqlens, s0, heads=heads)
    if norm:
        out = OL.gated_rmsnorm(out, z, L.norm_w, 1e-6)
        if heads is not None:
            mask = np.zeros(case.H_v, bool)
            mask[list(heads)] = True
            out[:, ~mask] = 0.0
    return out, sf, None


def compare_layer(case, L, out, pool_out, ref, conv=True, heads=None, tol=None):
    """Output and states to the tolerance; convolution states bit-exact (they
    are copies of inputs)."""
    ref_out, ref_state, ref_conv = ref
    tol = tol or TOL[case.dtype]
    hs = list(range(case.H_v)) if heads is None else list(heads)
    assert bool(torch.isfinite(out.float()).all()), "non-finite output"
    o = out[:, hs].float().cpu().numpy().astype(np.float64)
    eo, _ = rel_err(o, ref_out[:, hs], bf16_out=out.dtype == torch.bfloat16)
    if conv:
        cs, st = split_pool(case, L, pool_out)
    else:
        cs, st = None, pool_out.cpu().numpy()
    sl = [int(case.slot_out[i]) for i in range(case.n_seqs)]
    es, _ = rel_err(st[sl][:, hs].astype(np.float64), ref_state[:, hs])
    say(f"  {case.name}: out err/rms = {eo:.3e}, state err/rms = {es:.3e} (tol {tol:g})")
    assert eo <= tol, f"output error {eo:.3e} > {tol}"
    assert es <= tol, f"state error {es:.3e} > {tol}"
    if conv:
        got = cs[sl].astype(np.float64)
        assert np.array_equal(got, ref_conv), \
            f"convolution state differs at {np.argwhere(got != ref_conv)[:4].tolist()}"
    return eo, es
