"""GPU parity of gdn_recurrent_multi (several tokens per sequence, recurrent
form, state held on chip for the whole call) against the fp64 oracle.

Covers the speculative-verification shape (64 sequences x 4 and x 16 tokens,
Qwen3-Next heads), weak decay (so the state carried from token to token is
visible), ragged lengths including empty sequences over head-dim / head-ratio
/ dtype combinations, the zero-state slot, out-of-place state with untouched
slots, and agreement with gdn_chunked_prefill and gdn_recurrent_step."""
import numpy as np
import pytest
import torch

import workloads as gi
from gpu_harness import (TOL, compare_prefill, dev_case, gpu_decode_multi, gpu_prefill,
                         oracle_case, rel_err, say)

pytestmark = pytest.mark.gpu


def _check(case, inplace=True, out_dtype=torch.float32, heads=None):
    say(f"decode_multi {case.name}: N={case.n_seqs} T={case.total_tokens} H_k={case.H_k} "
        f"H_v={case.H_v} d_k={case.d_k} d_v={case.d_v} {case.dtype} out={out_dtype}")
    out, pool = gpu_decode_multi(case, inplace=inplace, out_dtype=out_dtype)
    ref_o, ref_s = oracle_case(case, heads=heads)
    return compare_prefill(case, out, pool, ref_o, ref_s, heads=heads)


@pytest.mark.parametrize("tokens", [2, 4, 16])
def test_speculative_batch_qwen_heads(tokens):
    case = gi.make_case(f"spec64x{tokens}", [tokens] * 64, dtype="bf16", seed=40 + tokens,
                        n_slots=64, scatter_slots=True, **gi.QWEN3_NEXT_HEADS)
    _check(case)


def test_speculative_batch_bf16_output():
    case = gi.make_case("spec64x4_bf16out", [4] * 64, dtype="bf16", seed=47,
                        **gi.QWEN3_NEXT_HEADS)
    _check(case, out_dtype=torch.bfloat16)


def test_weak_decay_carry():
    case = gi.make_case("spec8x16_weak", [16] * 8, dtype="bf16", seed=48, decay="weak",
                        **gi.QWEN3_NEXT_HEADS)
    _check(case)


@pytest.mark.parametrize("H_k,H_v,d_k,d_v,dtype", [
    (2, 2, 32, 32, "f32"), (1, 4, 64, 32, "f32"), (2, 4, 32, 128, "bf16"),
    (4, 4, 128, 64, "bf16"), (1, 2, 128, 128, "f32"), (2, 8, 64, 128, "bf16"),
])
def test_ragged_lengths(H_k, H_v, d_k, d_v, dtype):
    lengths = [0, 1, 2, 3, 5, 8, 13, 16, 31, 70]
    case = gi.make_case(f"ragged_{H_k}_{H_v}_{d_k}_{d_v}_{dtype}", lengths, H_k, H_v, d_k, d_v,
                        dtype, seed=49, decay="weak", n_slots=12, scatter_slots=True)
    _check(case)


def test_zero_state_and_untouched_slots():
    case = gi.make_case("zero_state", [3, 0, 7, 1], dtype="f32", seed=50, s0_std=0.0,
                        n_slots=9, scatter_slots=True, H_k=2, H_v=4, d_k=64, d_v=64)
    _check(case, inplace=False)
    d = dev_case(case)
    keep = d["pool"].clone()
    _, pool = gpu_decode_multi(case, d=d, inplace=False)
    written = set(int(x) for x in case.slot_out)
    for s in range(case.pool.shape[0]):
        if s not in written:
            assert torch.equal(pool[s], keep[s]), f"slot {s} changed"


def test_agrees_with_chunked_prefill_and_single_step():
    case = gi.make_case("agree", [5] * 16, dtype="bf16", seed=51, decay="weak",
                        **gi.QWEN3_NEXT_HEADS)
    d = dev_case(case)
    o_m, s_m = gpu_decode_multi(case, d=d, inplace=False)
    o_p, s_p = gpu_prefill(case, d=d, inplace=False)
    e_o, _ = rel_err(o_m.cpu().numpy(), o_p.cpu().numpy())
    e_s, _ = rel_err(s_m.cpu().numpy(), s_p.cpu().numpy())
    say(f"  multi vs chunked prefill: out {e_o:.2e}, state {e_s:.2e}")
    assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"]
    # one token per sequence: the same arithmetic as gdn_recurrent_step
    import gated_deltanet_rule_amd as gdn
    one = gi.make_case("one", [1] * 32, dtype="bf16", seed=52, **gi.QWEN3_NEXT_HEADS)
    d1 = dev_case(one)
    o1, s1 = gpu_decode_multi(one, d=d1, inplace=False)
    o2 = torch.empty_like(o1)
    s2 = d1["pool"].clone()
    gdn.decode_step(d1["q"], d1["k"], d1["v"], d1["g"], d1["beta"], d1["pool"], s2, o2,
                    d1["slot_in"], d1["slot_out"])
    torch.cuda.synchronize()
    assert torch.allclose(o1, o2, rtol=1e-5, atol=1e-6)
    assert torch.allclose(s1, s2, rtol=1e-5, atol=1e-6)


def test_f32_inputs_bf16_output():
    case = gi.make_case("multi_f32_bf16out", [0, 1, 3, 7, 16], 2, 4, 128, 32, "f32", seed=96,
                        decay="weak", n_slots=6, scatter_slots=True)
    _check(case, out_dtype=torch.bfloat16)
