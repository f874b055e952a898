"""GPU parity of the layer fusion against the fp64 oracle (oracle.layer):
the causal-convolution + SiLU prologue (mixed q|k|v rows, convolution state
at the start of each slot row) and the gated RMSNorm epilogue, through the
chunked prefill, the single-token step and the multi-token call.

Outputs and recurrent states are held to the operator's tolerance; the new
convolution states are copies of inputs and must match bit for bit.  Covers
the named head shapes, ragged and very short sequences (whose new
convolution state mixes the old state and the new rows), the zero-state
slot, empty sequences, untouched slots, out-of-place pools, a sequence fed in
several calls, the prefill -> step hand-off, each fusion on its own, and the
split-phase scan with the epilogue."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as gi
from gpu_harness import (TOL, compare_layer, dev_layer, gpu_layer_multi, gpu_layer_prefill,
                         layer_pool, oracle_layer, rel_err, say, split_pool)

pytestmark = pytest.mark.gpu


def _layer(case, seed):
    return gi.make_layer_inputs(case.total_tokens, case.pool.shape[0], case.H_k, case.H_v,
                                case.d_k, case.d_v, case.dtype, seed)


def _prefill(case, L, conv=True, norm=True, raw_gates=False, heads=None, out_dtype=torch.float32,
             inplace=True, chunks=None):
    say(f"layer prefill {case.name}: N={case.n_seqs} T={case.total_tokens} H_v={case.H_v} "
        f"{case.dtype} conv={conv} norm={norm} raw_gates={raw_gates} chunks={chunks}")
    out, pool = gpu_layer_prefill(case, L, conv, norm, raw_gates, out_dtype, inplace, chunks)
    ref = oracle_layer(case, L, conv, norm, raw_gates, heads)
    compare_layer(case, L, out, pool, ref, conv, heads)
    return out, pool


def test_prefill_conv_norm_tiny_f32():
    case = gi.make_case("layer_tiny", [128], 2, 2, 32, 32, "f32", seed=80)
    _prefill(case, _layer(case, 80))


def test_prefill_layer_varlen_in_ranges_bf16():
    """A fused-layer batch whose two-term factors (3.5 MiB per chunk) run as
    three chunk ranges, with sequences that cross range boundaries: the
    convolution history of a range's first chunk comes from the preceding
    rows, of a sequence's first chunk from its slot (sampled heads)."""
    case = gi.make_case("layer_ranges", [3000, 1500, 1, 700], dtype="bf16", seed=89,
                        decay="weak", n_slots=6, scatter_slots=True, **gi.QWEN3_NEXT_HEADS)
    _prefill(case, _layer(case, 89), raw_gates=True, heads=[0, 17, 31])


@pytest.mark.parametrize("H_k,H_v,dtype", [(2, 2, "bf16"), (1, 4, "bf16"), (1, 8, "f32")])
def test_prefill_layer_head_ratios_d128(H_k, H_v, dtype):
    """The fused prefill at d_k = d_v = 128 (the eight-wave two-term or fp32
    preparation) at head ratios other than 2, ragged lengths, raw gates."""
    case = gi.make_case(f"layer_ratio_{H_k}_{H_v}_{dtype}", [1, 63, 64, 65, 200], H_k, H_v, 128,
                        128, dtype, seed=97 + H_v, decay="weak", n_slots=8, scatter_slots=True)
    _prefill(case, _layer(case, 97 + H_v), raw_gates=True)


def test_prefill_conv_ragged_short_sequences_f32():
    case = gi.make_case("layer_ragged", [1, 2, 3, 63, 64, 65, 130], 2, 4, 64, 32, "f32", seed=81,
                        decay="weak", n_slots=12, scatter_slots=True)
    slot_in = case.slot_in.copy()
    slot_in[2] = -1                                   # one sequence starts from zero states
    case = dataclasses.replace(case, slot_in=slot_in)
    _prefill(case, _layer(case, 81), norm=False)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_prefill_layer_T4096_bf16(out_dtype):
    case = gi.config1()
    _prefill(case, _layer(case, 1), raw_gates=True, heads=[0, 9, 22, 31], out_dtype=out_dtype)


def test_prefill_layer_varlen_bf16():
    case = gi.config3()
    _prefill(case, _layer(case, 3), heads=[0, 13, 31])


def test_prefill_layer_streamed_weak_decay():
    case = gi.make_case("layer_stream", [1000], dtype="bf16", seed=82, decay="weak",
                        **gi.QWEN3_NEXT_HEADS)
    _prefill(case, _layer(case, 82), heads=[1, 30], chunks=256)


def test_prefill_out_of_place_equals_in_place_and_untouched_slots():
    case = gi.make_case("layer_slots", [0, 5, 70], 2, 4, 32, 64, "bf16", seed=83, n_slots=9,
                        scatter_slots=True)
    L = _layer(case, 83)
    o1, p1 = gpu_layer_prefill(case, L, inplace=True)
    o2, p2 = gpu_layer_prefill(case, L, inplace=False)
    assert torch.equal(o1, o2) and torch.equal(p1, p2)
    rows = layer_pool(case, L)
    owned = set(int(s) for s in case.slot_out)
    P = p1.cpu().numpy()
    for s in range(rows.shape[0]):
        if s not in owned:
            assert np.array_equal(P[s], rows[s])
    compare_layer(case, L, o1, p1, oracle_layer(case, L))


def test_norm_only_prefill_and_split_phase():
    import gated_deltanet_rule_amd as gdn
    case = gi.make_case("norm_only", [200, 77], 2, 4, 64, 64, "f32", seed=84, n_slots=2)
    L = _layer(case, 84)
    _prefill(case, L, conv=False)
    # split phase: the epilogue runs with the scan
    d = dev_layer(case, L, conv=False)
    out = torch.empty(d["v"].shape, dtype=torch.float32, device="cuda")
    plan = gdn.PrefillPlan(d["q"], d["v"], out, case.n_seqs, state=d["pool"], z=d["z"],
                           norm_w=d["norm_w"])
    plan.prepare(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"])
    plan.scan(d["pool"], d["pool"], out, d["slot_in"], d["slot_out"])
    torch.cuda.synchronize()
    compare_layer(case, L, out, d["pool"], oracle_layer(case, L, conv=False), conv=False)


def _decode_steps(dc, L, conv=True, norm=True, raw_gates=False):
    """Run a decode workload step by step through gdn.decode_step with the
    layer fusion; returns (out [S, N, H_v, d_v], slot rows)."""
    import gated_deltanet_rule_amd as gdn
    dt = torch.bfloat16 if dc.dtype == "bf16" else torch.float32
    f = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(t)
    S, N = dc.n_steps, dc.n_seqs
    C = L.qkv.shape[1]
    qkv = f(L.qkv.reshape(S, N, C), dt)
    z = f(L.z.reshape(S, N, dc.H_v, dc.d_v), dt) if norm else None
    n = dc.pool.shape[0]
    pool = f(np.concatenate([L.conv_pool.reshape(n, -1), dc.pool.reshape(n, -1)], axis=1)) if conv \
        else f(dc.pool)
    g, b = (f(dc.raw_a), f(dc.raw_b)) if raw_gates else (f(dc.g), f(dc.beta))
    gates = (f(dc.ssm_a), f(dc.ssm_dt)) if raw_gates else None
    q, k, v = f(dc.q, dt), f(dc.k, dt), f(dc.v, dt)
    slots = f(dc.slots, torch.int32)
    outs = torch.empty((S, N, dc.H_v, dc.d_v), dtype=torch.float32, device="cuda")
    cw = f(L.conv_w)
    nw = f(L.norm_w)
    for s in range(S):
        if conv:
            gdn.decode_step(qkv[s], None, None, g[s], b[s], pool, pool, outs[s], slots, slots,
                            gates=gates, conv=(cw, dc.H_k, dc.d_k), z=z[s] if norm else None,
                            norm_w=nw if norm else None)
        else:
            gdn.decode_step(q[s], k[s], v[s], g[s], b[s], pool, pool, outs[s], slots, slots,
                            gates=gates, z=z[s] if norm else None, norm_w=nw if norm else None)
    torch.cuda.synchronize()
    return outs, pool


def _decode_as_case(dc, L):
    """The same decode workload as N sequences of n_steps tokens (oracle side)."""
    S, N = dc.n_steps, dc.n_seqs
    perm = lambda a: np.ascontiguousarray(np.swapaxes(a.reshape((S, N) + a.shape[1:]), 0, 1)).reshape(
        (S * N,) + a.shape[1:])
    q, k, v, g, b, cu = gi.decode_as_sequences(dc)
    sw = lambda a: np.ascontiguousarray(np.swapaxes(a, 0, 1)).reshape((S * N,) + a.shape[2:])
    case = gi.Case(dc.name, dc.H_k, dc.H_v, dc.d_k, dc.d_v, dc.dtype, [S] * N, q, k, v, g, b,
                   dc.pool, dc.slots.copy(), dc.slots.copy(), dc.ssm_a, sw(dc.raw_a), sw(dc.raw_b),
                   dc.ssm_dt)
    Lc = dataclasses.replace(L, qkv=perm(L.qkv), z=perm(L.z))
    return case, Lc


@pytest.mark.parametrize("conv,norm", [(True, True), (True, False), (False, True)])
def test_decode_step_layer_qwen_heads(conv, norm):
    dc = gi.make_decode("layer_decode", 16, 6, dtype="bf16", seed=85, **gi.QWEN3_NEXT_HEADS)
    L = gi.make_layer_inputs(16 * 6, 16, dc.H_k, dc.H_v, dc.d_k, dc.d_v, "bf16", 85)
    say(f"layer decode: 16 x 6 steps conv={conv} norm={norm}")
    outs, pool = _decode_steps(dc, L, conv, norm, raw_gates=True)
    case, Lc = _decode_as_case(dc, L)
    heads = [0, 9, 22, 31]
    ref_o, ref_s, ref_c = oracle_layer(case, Lc, conv, norm, raw_gates=True, heads=heads)
    # [N*S] sequence-major -> [S, N]
    ref_o = ref_o.reshape(dc.n_seqs, dc.n_steps, dc.H_v, dc.d_v).swapaxes(0, 1)
    o = outs.cpu().numpy().astype(np.float64)
    eo, _ = rel_err(o[:, :, heads], ref_o[:, :, heads])
    if conv:
        cs, st = split_pool(case, Lc, pool)
    else:
        cs, st = None, pool.cpu().numpy()
    es, _ = rel_err(st[dc.slots][:, heads].astype(np.float64), ref_s[:, heads])
    say(f"  out err/rms = {eo:.3e}, state err/rms = {es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    if conv:
        assert np.array_equal(cs[dc.slots].astype(np.float64), ref_c)


def test_decode_step_layer_f32_tight():
    dc = gi.make_decode("layer_decode_f32", 4, 9, 1, 2, 64, 32, "f32", seed=86, decay="weak")
    L = gi.make_layer_inputs(4 * 9, 4, 1, 2, 64, 32, "f32", 86)
    outs, pool = _decode_steps(dc, L)
    case, Lc = _decode_as_case(dc, L)
    ref_o, ref_s, ref_c = oracle_layer(case, Lc)
    ref_o = ref_o.reshape(4, 9, 2, 32).swapaxes(0, 1)
    eo, _ = rel_err(outs.cpu().numpy(), ref_o)
    cs, st = split_pool(case, Lc, pool)
    es, _ = rel_err(st[dc.slots].astype(np.float64), ref_s)
    say(f"  f32 decode layer: out {eo:.3e} state {es:.3e}")
    assert eo <= TOL["f32"] and es <= TOL["f32"]
    assert np.array_equal(cs[dc.slots].astype(np.float64), ref_c)


@pytest.mark.parametrize("H_k,H_v", [(2, 2), (1, 4)])
def test_decode_step_layer_head_ratios(H_k, H_v):
    """The prologue at head ratios 1 (one value head per workgroup, state
    replaced by the decode kernel) and 4 (state replaced by the separate
    pass), with in-place pools."""
    dc = gi.make_decode("layer_ratio", 5, 4, H_k, H_v, 64, 64, "f32", seed=90, decay="weak")
    L = gi.make_layer_inputs(5 * 4, 5, H_k, H_v, 64, 64, "f32", 90)
    say(f"layer decode ratios H_k={H_k} H_v={H_v}")
    outs, pool = _decode_steps(dc, L)
    case, Lc = _decode_as_case(dc, L)
    ref_o, ref_s, ref_c = oracle_layer(case, Lc)
    ref_o = ref_o.reshape(5, 4, H_v, 64).swapaxes(0, 1)
    eo, _ = rel_err(outs.cpu().numpy(), ref_o)
    cs, st = split_pool(case, Lc, pool)
    es, _ = rel_err(st[dc.slots].astype(np.float64), ref_s)
    assert eo <= TOL["f32"] and es <= TOL["f32"]
    assert np.array_equal(cs[dc.slots].astype(np.float64), ref_c)


@pytest.mark.parametrize("H_k,H_v", [(2, 2), (1, 4)])
def test_multi_layer_head_ratios(H_k, H_v):
    case = gi.make_case("layer_multi_ratio", [0, 1, 3, 9], H_k, H_v, 64, 64, "f32", seed=91,
                        decay="weak", n_slots=6, scatter_slots=True)
    L = _layer(case, 91)
    out, pool = gpu_layer_multi(case, L)
    compare_layer(case, L, out, pool, oracle_layer(case, L))


def test_multi_layer_speculative_qwen_heads():
    case = gi.make_case("layer_spec64x4", [4] * 64, dtype="bf16", seed=87, n_slots=64,
                        scatter_slots=True, **gi.QWEN3_NEXT_HEADS)
    L = _layer(case, 87)
    out, pool = gpu_layer_multi(case, L, raw_gates=True)
    compare_layer(case, L, out, pool, oracle_layer(case, L, raw_gates=True, heads=[0, 5, 31]),
                  heads=[0, 5, 31])


@pytest.mark.parametrize("conv,norm", [(True, True), (True, False), (False, True)])
def test_multi_layer_ragged_f32(conv, norm):
    case = gi.make_case("layer_multi", [0, 1, 2, 5, 16], 1, 2, 128, 64, "f32", seed=88,
                        decay="weak", n_slots=7, scatter_slots=True)
    L = _layer(case, 88)
    out, pool = gpu_layer_multi(case, L, conv, norm)
    compare_layer(case, L, out, pool, oracle_layer(case, L, conv, norm), conv)


def test_prefill_then_steps_equals_one_sequence():
    """prefill of T - n tokens, then n single-token steps, with the
    convolution state carried in the slot rows == the oracle over T tokens."""
    import gated_deltanet_rule_amd as gdn
    T, n = 150, 5
    case = gi.make_case("layer_handoff", [T], 2, 4, 64, 64, "bf16", seed=89, decay="weak")
    L = _layer(case, 89)
    d = dev_layer(case, L)
    out = torch.empty((T, case.H_v, case.d_v), dtype=torch.float32, device="cuda")
    cv = (d["conv_w"], case.H_k, case.d_k)
    cu = torch.tensor([0, T - n], dtype=torch.int32, device="cuda")
    gdn.prefill(d["qkv"][:T - n], None, None, d["g"][:T - n], d["beta"][:T - n], d["pool"], d["pool"],
                out[:T - n], cu, d["slot_in"], d["slot_out"], conv=cv, z=d["z"][:T - n], norm_w=d["norm_w"])
    for t in range(T - n, T):
        gdn.decode_step(d["qkv"][t:t + 1], None, None, d["g"][t:t + 1], d["beta"][t:t + 1], d["pool"],
                        d["pool"], out[t:t + 1], d["slot_out"], d["slot_out"], conv=cv, z=d["z"][t:t + 1],
                        norm_w=d["norm_w"])
    torch.cuda.synchronize()
    compare_layer(case, L, out, d["pool"], oracle_layer(case, L))


def test_norm_only_bf16_output_is_rounded_once():
    """bf16 q/k/v and output with the epilogue alone: o is kept in fp32 up to
    the norm, so the only rounding is the final one."""
    case = gi.config1(2048)
    _prefill(case, _layer(case, 90), conv=False, heads=[3, 17], out_dtype=torch.bfloat16)


@pytest.mark.parametrize("tokens", [1, 3])
@pytest.mark.parametrize("no_pool", [False, True])
def test_fused_decode_fresh_slots(tokens, no_pool):
    """The fused recurrent kernels at Qwen3-Next heads (two value heads per
    workgroup, convolution state replaced in place by the workgroup): one
    token per sequence through gdn_recurrent_step, three through
    gdn_recurrent_multi.  Sequences whose input slot is -1, and with no input
    pool every sequence, start from zero recurrent and convolution states
    (both read through empty ranges); outputs are written to other slots.
    Against the oracle with the same starting states."""
    import gated_deltanet_rule_amd as gdn
    case = gi.make_case("layer_fresh", [tokens] * 8, dtype="bf16", seed=95, n_slots=16,
                        scatter_slots=True, **gi.QWEN3_NEXT_HEADS)
    slot_in = case.slot_in.copy()
    if no_pool:
        slot_in[:] = -1
    else:
        slot_in[1] = slot_in[5] = -1
    case = dataclasses.replace(case, slot_in=slot_in)
    L = _layer(case, 95)
    say(f"fused decode fresh slots: tokens={tokens} no_pool={no_pool}")
    d = dev_layer(case, L)
    out = torch.empty((case.total_tokens, case.H_v, case.d_v), dtype=torch.float32, device="cuda")
    pool_out = d["pool"].clone()
    pool_in = None if no_pool else d["pool"]
    si = torch.from_numpy(slot_in).cuda()
    args = dict(gates=(d["ssm_a"], d["ssm_dt"]), conv=(d["conv_w"], case.H_k, case.d_k), z=d["z"],
                norm_w=d["norm_w"])
    if tokens == 1:
        gdn.decode_step(d["qkv"], None, None, d["raw_a"], d["raw_b"], pool_in, pool_out, out, si,
                        d["slot_out"], **args)
    else:
        gdn.decode_multi(d["qkv"], None, None, d["raw_a"], d["raw_b"], pool_in, pool_out, out, d["cu"],
                         si, d["slot_out"], **args)
    torch.cuda.synchronize()
    heads = [0, 17, 31]
    compare_layer(case, L, out, pool_out, oracle_layer(case, L, raw_gates=True, heads=heads), heads=heads)
