"""GPU parity of the in-kernel gate activations (gate_mode GDN_GATES_RAW):
g = softplus(a + ssm_dt) * ssm_a and beta = sigmoid(b) computed inside the
kernels from the raw projections a, b, against the fp64 oracle fed with the
same activations evaluated in fp64.

Covers every entry point (chunked prefill, single-token recurrent step,
multi-token recurrent call), the named workload shapes, weak decay (so a gate
error would accumulate through the carried state), and raw projections far
into both tails (softplus near the identity and near zero, sigmoid saturated).
The named workloads run exactly as stated (raw a, b ~ N(0, 1), no gate bias);
the stress cases add a per-head gate bias ssm_dt ~ U(-1, 1)."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as gi
from gpu_harness import (compare_decode, compare_prefill, gpu_decode_multi, gpu_prefill,
                         oracle_case, oracle_decode, run_decode, say)

pytestmark = pytest.mark.gpu


def _prefill(case, heads=None, out_dtype=torch.float32):
    say(f"prefill raw gates {case.name}: N={case.n_seqs} T={case.total_tokens} "
        f"H_v={case.H_v} {case.dtype}")
    out, pool = gpu_prefill(case, out_dtype=out_dtype, raw_gates=True)
    ref_o, ref_s = oracle_case(case, heads=heads, raw_gates=True)
    return compare_prefill(case, out, pool, ref_o, ref_s, heads=heads)


def _multi(case, heads=None):
    say(f"decode_multi raw gates {case.name}: N={case.n_seqs} T={case.total_tokens}")
    out, pool = gpu_decode_multi(case, raw_gates=True)
    ref_o, ref_s = oracle_case(case, heads=heads, raw_gates=True)
    return compare_prefill(case, out, pool, ref_o, ref_s, heads=heads)


def _scaled(case, sa, sb):
    """The same case with the raw projections stretched into the tails."""
    return dataclasses.replace(case, name=f"{case.name}_x{sa:g}_{sb:g}",
                               raw_a=(case.raw_a * sa).astype(np.float32),
                               raw_b=(case.raw_b * sb).astype(np.float32))


def test_prefill_tiny_f32():
    _prefill(gi.config0())


def test_prefill_T4096_bf16():
    _prefill(gi.config1())


def test_prefill_weak_decay_ragged_f32():
    case = gi.make_case("gates_weak", [1, 63, 64, 65, 200], 2, 4, 64, 64, "f32", seed=71,
                        decay="weak", gate_bias=True, n_slots=8, scatter_slots=True)
    _prefill(case)


def test_prefill_varlen_bf16_output():
    _prefill(gi.config3(), out_dtype=torch.bfloat16)


@pytest.mark.parametrize("sa,sb", [(30.0, 40.0), (0.05, 0.05)])
def test_prefill_tails(sa, sb):
    case = gi.make_case("gates_tails", [130, 64], 2, 4, 128, 128, "f32", seed=72,
                        decay="weak", gate_bias=True)
    _prefill(_scaled(case, sa, sb))


def test_recurrent_step_qwen_heads():
    dc = gi.make_decode("gates_decode", 16, 8, dtype="bf16", seed=73, **gi.QWEN3_NEXT_HEADS)
    heads = [0, 9, 22, 31]
    outs, pool = run_decode(dc, raw_gates=True)
    ref_o, ref_s = oracle_decode(dc, heads=heads, raw_gates=True)
    compare_decode(dc, outs, pool, ref_o, ref_s, heads=heads)


def test_recurrent_step_weak_decay_tails_f32():
    dc = gi.make_decode("gates_decode_tails", 4, 12, 2, 4, 64, 128, "f32", seed=74,
                        decay="weak", gate_bias=True)
    dc = dataclasses.replace(dc, raw_a=(dc.raw_a * 25).astype(np.float32),
                             raw_b=(dc.raw_b * 30).astype(np.float32))
    outs, pool = run_decode(dc, raw_gates=True)
    ref_o, ref_s = oracle_decode(dc, raw_gates=True)
    compare_decode(dc, outs, pool, ref_o, ref_s)


def test_multi_speculative_qwen_heads():
    case = gi.make_case("gates_spec64x4", [4] * 64, dtype="bf16", seed=75, n_slots=64,
                        scatter_slots=True, **gi.QWEN3_NEXT_HEADS)
    _multi(case)


def test_multi_weak_decay_ragged_tails():
    case = gi.make_case("gates_multi", [0, 1, 5, 16, 3], 1, 2, 128, 64, "f32", seed=76,
                        decay="weak", gate_bias=True)
    _multi(_scaled(case, 20.0, 20.0))


def test_multi_raw_gates_past_64_tokens():
    """The multi-token kernel activates the raw gates of 64 tokens at a time
    per wave: sequences that cross one and two such batches."""
    case = gi.make_case("gates_multi_long", [65, 0, 130, 2, 64], 1, 2, 128, 64, "bf16", seed=77,
                        decay="weak", gate_bias=True)
    _multi(case)


def test_raw_gates_match_precomputed_gates():
    """The raw path and the final-gate path on the same tokens agree: the
    kernels' fp32 activations differ from torch's fp32 ones only by rounding."""
    case = gi.make_case("gates_vs_final", [100, 300], 2, 4, 64, 64, "f32", seed=77,
                        decay="weak", gate_bias=True)
    a = torch.from_numpy(case.raw_a).double()
    b = torch.from_numpy(case.raw_b).double()
    g = torch.nn.functional.softplus(a + torch.from_numpy(case.ssm_dt).double()) \
        * torch.from_numpy(case.ssm_a).double()
    fin = dataclasses.replace(case, g=g.float().numpy(), beta=torch.sigmoid(b).float().numpy())
    o_raw, s_raw = gpu_prefill(case, raw_gates=True)
    o_fin, s_fin = gpu_prefill(fin)
    scale_o = float(o_fin.double().pow(2).mean().sqrt())
    scale_s = float(s_fin.double().pow(2).mean().sqrt())
    eo = float((o_raw.double() - o_fin.double()).abs().max()) / scale_o
    es = float((s_raw.double() - s_fin.double()).abs().max()) / scale_s
    say(f"  raw vs final gates: out {eo:.3e}, state {es:.3e}")
    assert eo <= 1e-4 and es <= 1e-4
