"""Every compiled head-dimension / input-type combination against the fp64 oracle.

The kernels are instantiated for d_k, d_v in {32, 64, 128} and for fp32 and
bf16 inputs; each of the 18 combinations runs here through the chunked
prefill (ragged lengths, one empty sequence, a ragged final chunk), the
single-token step, the multi-token call, and the fused layer prefill (causal
convolution + SiLU prologue, in-kernel gate activations, gated RMSNorm
epilogue).  Two key heads serve four value heads, so the head grouping is
exercised everywhere; slots are scattered over a larger pool."""
import itertools

import pytest
import torch

import workloads as gi
from gpu_harness import (compare_decode, compare_layer, compare_prefill, gpu_decode_multi,
                         gpu_layer_prefill, gpu_prefill, oracle_case, oracle_decode, oracle_layer,
                         run_decode, say)

pytestmark = pytest.mark.gpu

DIMS = [32, 64, 128]
COMBOS = [(dk, dv, dt) for dk, dv in itertools.product(DIMS, DIMS) for dt in ("f32", "bf16")]
IDS = [f"dk{dk}-dv{dv}-{dt}" for dk, dv, dt in COMBOS]


def _seed(d_k, d_v, dtype, salt):
    return 1000 + 7 * d_k + 3 * d_v + (1 if dtype == "bf16" else 0) + 100 * salt


@pytest.mark.parametrize("d_k,d_v,dtype", COMBOS, ids=IDS)
def test_prefill(d_k, d_v, dtype):
    case = gi.make_case(f"sweep_prefill_{d_k}_{d_v}_{dtype}", [0, 1, 63, 65, 130], 2, 4, d_k,
                        d_v, dtype, seed=_seed(d_k, d_v, dtype, 1), decay="custom", a_lo=0.02,
                        a_hi=0.3, n_slots=9, scatter_slots=True)
    say(f"prefill {case.name}: T={case.total_tokens}")
    out, pool = gpu_prefill(case)
    ref_o, ref_s = oracle_case(case)
    compare_prefill(case, out, pool, ref_o, ref_s)


@pytest.mark.parametrize("d_k,d_v,dtype", COMBOS, ids=IDS)
def test_decode_step(d_k, d_v, dtype):
    dc = gi.make_decode(f"sweep_step_{d_k}_{d_v}_{dtype}", 5, 3, 2, 4, d_k, d_v, dtype,
                        seed=_seed(d_k, d_v, dtype, 2), decay="weak", n_slots=11,
                        scatter_slots=True)
    say(f"decode step {dc.name}: N={dc.n_seqs} steps={dc.n_steps}")
    outs, pool = run_decode(dc)
    ref_o, ref_s = oracle_decode(dc)
    compare_decode(dc, outs, pool, ref_o, ref_s)


@pytest.mark.parametrize("d_k,d_v,dtype", COMBOS, ids=IDS)
def test_decode_multi(d_k, d_v, dtype):
    case = gi.make_case(f"sweep_multi_{d_k}_{d_v}_{dtype}", [3, 0, 1, 16, 5], 2, 4, d_k, d_v,
                        dtype, seed=_seed(d_k, d_v, dtype, 3), decay="weak", n_slots=8,
                        scatter_slots=True)
    say(f"decode multi {case.name}: T={case.total_tokens}")
    out, pool = gpu_decode_multi(case)
    ref_o, ref_s = oracle_case(case)
    compare_prefill(case, out, pool, ref_o, ref_s)


@pytest.mark.parametrize("d_k,d_v,dtype", COMBOS, ids=IDS)
def test_layer_prefill(d_k, d_v, dtype):
    case = gi.make_case(f"sweep_layer_{d_k}_{d_v}_{dtype}", [2, 64, 97], 2, 4, d_k, d_v, dtype,
                        seed=_seed(d_k, d_v, dtype, 4), decay="weak", n_slots=6,
                        scatter_slots=True)
    L = gi.make_layer_inputs(case.total_tokens, case.pool.shape[0], case.H_k, case.H_v,
                             case.d_k, case.d_v, case.dtype, _seed(d_k, d_v, dtype, 4))
    say(f"layer prefill {case.name}: T={case.total_tokens}")
    out, pool = gpu_layer_prefill(case, L, conv=True, norm=True, raw_gates=True,
                                  out_dtype=torch.float32, inplace=True, chunks=None)
    ref = oracle_layer(case, L, conv=True, norm=True, raw_gates=True)
    compare_layer(case, L, out, pool, ref, conv=True)
