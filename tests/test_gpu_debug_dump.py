"""GDN_DEBUG_DUMP: the library's record of one chunk's intermediates (G, T,
W = k_cumdecay, U = v_new) against the oracle's chunk record on the same
inputs.  Bounds: G is the same fp64 cumulative sum of the same fp32 gates; T
is formed in fp32 from exact bf16 products by substitution (held to 1e-6 of
max|T|; measured up to 5e-8), W from two-term bf16 operands (16 significant
bits: held to 5e-5 of max|W|; measured up to 4e-6); U carries the rounding of
W to a bf16 operand in the scan (2^-9 relative) and the state carried from
earlier chunks, and is held to the output bound of the bf16 parity tests
(measured 2e-5 in a sequence's second chunk, 3e-3 after 70 chunks)."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as gi
from gpu_harness import TOL, dev_case, gpu_prefill, say

pytestmark = pytest.mark.gpu


@pytest.fixture
def dump_env():
    old = os.environ.get("GDN_DEBUG_DUMP")
    yield
    if old is None:
        os.environ.pop("GDN_DEBUG_DUMP", None)
    else:
        os.environ["GDN_DEBUG_DUMP"] = old


def _s0(case):
    return np.stack([case.pool[s] if s >= 0 else np.zeros_like(case.pool[0]) for s in case.slot_in])


def _compare(rec, ref, dtype):
    assert rec["prepared"] == 1 and rec["scanned"] == 1
    assert rec["t0"] == ref["t0"] and rec["len"] == ref["len"]
    for name, tol in (("G", 1e-12), ("T", 1e-6), ("W", 5e-5)):
        err = np.abs(rec[name] - ref[name]).max() / max(np.abs(ref[name]).max(), 1e-30)
        say(f"  {name}: max err {err:.2e} of max|ref|")
        assert err <= tol, name
    u_rms = np.sqrt(np.mean(ref["U"] ** 2))
    err = np.abs(rec["U"] - ref["U"]).max() / u_rms
    say(f"  U: max err {err:.2e} of rms(ref)")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype,dk,dv,seq,offset,head", [
    ("bf16", 128, 128, 1, 70, 3),     # second chunk of a middle sequence: S != 0
    ("bf16", 64, 128, 0, 3, 0),       # first chunk (state from the slot)
    ("f32", 64, 64, 2, 40, 2),        # partial last chunk
])
def test_debug_record_matches_oracle(dump_env, dtype, dk, dv, seq, offset, head):
    import gated_deltanet_rule_amd as gdn
    case = gi.make_case("dump", [100, 200, 41], 2, 4, dk, dv, dtype, seed=41, scatter_slots=True)
    cu = case.cu_seqlens.astype(np.int64)
    token = int(cu[seq] + offset)
    say(f"dump {dtype} dk={dk} dv={dv} token={token} head={head}")
    os.environ["GDN_DEBUG_DUMP"] = f"{token},{head}"
    gpu_prefill(case, inplace=False)
    rec = gdn.debug_dump()
    ref = oracle.chunk_dump(case.q, case.k, case.v, case.g, case.beta, cu, _s0(case), token=token, head=head)
    n_before = sum((int(cu[i + 1] - cu[i]) + 63) // 64 for i in range(seq))
    assert rec["chunk"] == n_before + offset // 64
    assert rec["token"] == token and rec["head"] == head and rec["d_k"] == dk and rec["d_v"] == dv
    _compare(rec, ref, dtype)


def test_debug_record_split_phase_and_outside(dump_env):
    """The prepare / scan pair records the same chunk as the single call, the
    record does not change the results, and a token past the batch leaves it
    unwritten."""
    import gated_deltanet_rule_amd as gdn
    case = gi.make_case("dump_split", [130, 90], 2, 4, 128, 128, "bf16", seed=42)
    d = dev_case(case)
    os.environ.pop("GDN_DEBUG_DUMP", None)
    out_ref, pool_ref = gpu_prefill(case, d=d, inplace=False)
    token = int(case.cu_seqlens[1] + 65)
    os.environ["GDN_DEBUG_DUMP"] = f"{token},1"
    out_1, pool_1 = gpu_prefill(case, d=d, inplace=False)
    assert torch.equal(out_1, out_ref) and torch.equal(pool_1, pool_ref)
    rec1 = gdn.debug_dump()
    out = torch.empty(d["v"].shape, device="cuda")
    pool = d["pool"].clone()
    plan = gdn.PrefillPlan(d["q"], d["v"], out, case.n_seqs, state=pool)
    plan.prepare(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"])
    plan.scan(d["pool"], pool, out, d["slot_in"], d["slot_out"])
    torch.cuda.synchronize()
    rec2 = gdn.debug_dump()
    assert rec1["prepared"] == rec2["prepared"] == 1 and rec1["scanned"] == rec2["scanned"] == 1
    for name in ("G", "T", "W", "U"):
        assert np.array_equal(rec1[name], rec2[name]), name
    os.environ["GDN_DEBUG_DUMP"] = f"{case.total_tokens},1"
    gpu_prefill(case, d=d, inplace=False)
    rec3 = gdn.debug_dump()
    assert rec3["prepared"] == 0 and rec3["scanned"] == 0 and rec3["chunk"] == -1


@pytest.mark.parametrize("chunk", [70, 128])
def test_debug_record_in_a_later_chunk_range(dump_env, chunk):
    """A 8229-token call runs as several chunk ranges (64 chunks each at
    these heads): the record of a chunk in the second range (chunk 70) and of
    the partial last chunk (128, 37 tokens), whose state entered through the
    ranges' carry, matches the oracle's."""
    import gated_deltanet_rule_amd as gdn
    case = gi.make_case("dump_ranges", [8229], dtype="bf16", seed=43, decay="weak", **gi.QWEN3_NEXT_HEADS)
    token, head = 64 * chunk + 5, 17
    os.environ["GDN_DEBUG_DUMP"] = f"{token},{head}"
    gpu_prefill(case, inplace=False)
    rec = gdn.debug_dump()
    ref = oracle.chunk_dump(case.q, case.k, case.v, case.g, case.beta, case.cu_seqlens.astype(np.int64),
                            _s0(case), token=token, head=head)
    assert rec["chunk"] == chunk
    _compare(rec, ref, "bf16")
