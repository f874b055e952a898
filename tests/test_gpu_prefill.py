"""GPU parity of gdn_chunked_prefill against the fp64 oracle.

The named workloads run at their full sizes with their stated gate recipe
(beta = sigmoid(N(0,1)), g = -exp(A_log) softplus(N(0,1))), every value head
compared element by element.  Stress sets make chunk-to-chunk state carry
visible (weak decay), cover ragged lengths around the chunk size, head-dim
and head-ratio combinations, beta = 0, g = 0 with beta = 1, zero-length
sequences, the zero-state slot, in-place vs out-of-place state, and the
prefill -> decode hand-off."""
import numpy as np
import pytest
import torch

import workloads as gi
import oracle
from gpu_harness import (TOL, compare_prefill, dev_case, gpu_prefill, oracle_case,
                         rel_err, say)

pytestmark = pytest.mark.gpu


def _check(case, heads=None, inplace=True, chunks=None, out_dtype=torch.float32):
    say(f"prefill {case.name}: N={case.n_seqs} T={case.total_tokens} H_k={case.H_k} "
        f"H_v={case.H_v} d_k={case.d_k} d_v={case.d_v} {case.dtype} chunks={chunks} "
        f"out={out_dtype}")
    out, pool = gpu_prefill(case, inplace=inplace, chunks=chunks, out_dtype=out_dtype)
    ref_o, ref_s = oracle_case(case, heads=heads)
    return compare_prefill(case, out, pool, ref_o, ref_s, heads=heads)


def test_tiny_f32_T128():
    _check(gi.config0())


def test_prefill_T4096_full():
    _check(gi.config1())


def test_prefill_T4096_bf16_output():
    _check(gi.config1(), out_dtype=torch.bfloat16)


def test_varlen_8_sequences_scattered_slots():
    _check(gi.config3())


def test_varlen_untouched_slots_and_out_of_place():
    case = gi.make_case("varlen_small", [17, 64, 65, 130], 2, 4, 64, 64, "bf16", seed=31,
                        n_slots=12, scatter_slots=True)
    out1, pool1 = gpu_prefill(case, inplace=True)
    out2, pool2 = gpu_prefill(case, inplace=False)
    assert torch.equal(out1, out2) and torch.equal(pool1, pool2)
    owned = set(int(s) for s in case.slot_out)
    P = pool1.cpu().numpy()
    for s in range(case.pool.shape[0]):
        if s not in owned:
            assert np.array_equal(P[s], case.pool[s])


def test_stream_65536_as_128_calls_of_512():
    _check(gi.config4(), chunks=512)


@pytest.mark.parametrize("shape", ["T4096", "stream8192"])
def test_weak_decay_state_carry(shape):
    if shape == "T4096":
        case = gi.make_case("weak_T4096", [4096], dtype="bf16", seed=41, decay="weak",
                            **gi.QWEN3_NEXT_HEADS)
        _check(case)
    else:
        case = gi.make_case("weak_stream8192", [8192], dtype="bf16", seed=42, decay="weak",
                            **gi.QWEN3_NEXT_HEADS)
        _check(case, heads=[0, 3, 16, 31], chunks=512)


def test_weak_decay_tiny_f32():
    _check(gi.make_case("weak_tiny_f32", [128], 2, 2, 32, 32, "f32", seed=43, decay="weak"))


LENGTHS = [1, 2, 63, 64, 65, 127, 128, 129, 0, 200]


@pytest.mark.parametrize("H_k,H_v,d_k,d_v,dtype", [
    (2, 2, 32, 32, "f32"), (1, 4, 64, 32, "f32"), (2, 4, 32, 128, "bf16"),
    (4, 4, 128, 64, "bf16"), (1, 2, 128, 128, "f32"), (2, 4, 128, 128, "bf16"),
    (1, 1, 64, 64, "bf16"), (2, 8, 64, 128, "bf16"),
    # d_k = d_v = 128 runs the eight-wave preparation, whose waves 4..7 repeat
    # the row scalars of waves 0..3: head ratios 1, 4 and 8 there
    (2, 2, 128, 128, "bf16"), (1, 4, 128, 128, "bf16"), (1, 8, 128, 128, "bf16"),
    (1, 8, 128, 128, "f32"),
])
def test_ragged_lengths_dims_and_ratios(H_k, H_v, d_k, d_v, dtype):
    case = gi.make_case(f"ragged_{H_k}_{H_v}_{d_k}_{d_v}_{dtype}", LENGTHS, H_k, H_v, d_k, d_v,
                        dtype, seed=d_k * 3 + d_v + H_v, decay="custom", a_lo=0.02, a_hi=0.3,
                        n_slots=16, scatter_slots=True)
    _check(case)


@pytest.mark.parametrize("mode", ["beta0", "g0_beta1", "zero_state"])
def test_degenerate_cases(mode):
    if mode == "beta0":
        case = gi.make_case("beta0", [150, 64], 2, 4, 64, 64, "f32", seed=51, beta_mode="zero",
                            decay="weak")
    elif mode == "g0_beta1":
        case = gi.make_case("g0_beta1", [100], 2, 2, 128, 128, "f32", seed=52, decay="zero",
                            beta_mode="one")
    else:
        case = gi.make_case("zero_state", [77, 3], 2, 4, 64, 64, "bf16", seed=53, s0_std=0.0)
    _check(case)


def test_strong_decay_outputs_finite_and_deterministic():
    case = gi.make_case("strong_T1024", [1024], dtype="bf16", seed=61, decay="custom",
                        a_lo=16.0, a_hi=64.0, **gi.QWEN3_NEXT_HEADS)
    d = dev_case(case)
    o1, p1 = gpu_prefill(case, d=d, inplace=False)
    o2, p2 = gpu_prefill(case, d=d, inplace=False)
    assert torch.isfinite(o1.float()).all() and torch.isfinite(p1).all()
    assert torch.equal(o1, o2) and torch.equal(p1, p2)


def test_split_phase_prefill_matches_single_call():
    """prepare on one stream, scan on another (ordered by an event) == one call."""
    import gated_deltanet_rule_amd as gdn
    case = gi.make_case("split", [200, 64, 1], 2, 4, 128, 128, "bf16", seed=81, decay="weak",
                        n_slots=5, scatter_slots=True)
    d = dev_case(case)
    out_ref, pool_ref = gpu_prefill(case, d=d, inplace=False)
    out = torch.empty(d["v"].shape, dtype=torch.float32, device="cuda")
    pool = d["pool"].clone()
    plan = gdn.PrefillPlan(d["q"], d["v"], out, case.n_seqs, state=pool)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ev = torch.cuda.Event()
    torch.cuda.synchronize()
    plan.prepare(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], stream=s1)
    ev.record(s1)
    s2.wait_event(ev)
    plan.scan(d["pool"], pool, out, d["slot_in"], d["slot_out"], stream=s2)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref) and torch.equal(pool, pool_ref)


def test_prefill_then_decode_equals_longer_prefill():
    """The state layout written by the prefill is the one the decode step reads:
    prefill(T - n) followed by n decode steps reproduces prefill(T)."""
    import gated_deltanet_rule_amd as gdn
    case = gi.make_case("handoff", [300], 2, 4, 128, 128, "bf16", seed=71, decay="weak")
    T, n = 300, 5
    d = dev_case(case)
    out_full, pool_full = gpu_prefill(case, d=d, inplace=False)
    pool = d["pool"].clone()
    out = torch.empty(d["v"].shape, dtype=torch.float32, device="cuda")
    cu = torch.tensor([0, T - n], dtype=torch.int32, device="cuda")
    gdn.prefill(d["q"][:T - n], d["k"][:T - n], d["v"][:T - n], d["g"][:T - n],
                d["beta"][:T - n], pool, pool, out[:T - n], cu, d["slot_in"], d["slot_out"])
    for t in range(T - n, T):
        gdn.decode_step(d["q"][t:t + 1], d["k"][t:t + 1], d["v"][t:t + 1], d["g"][t:t + 1],
                        d["beta"][t:t + 1], pool, pool, out[t:t + 1], d["slot_out"], d["slot_out"])
    torch.cuda.synchronize()
    ref_o, ref_s = oracle_case(case)
    compare_prefill(case, out, pool, ref_o, ref_s)
    e, _ = rel_err(out.cpu().numpy(), out_full.cpu().numpy())
    assert e <= TOL["bf16"]


def _split_phase(case, d):
    """prepare + scan as two calls: always one chunk range over the batch."""
    import gated_deltanet_rule_amd as gdn
    out = torch.empty(d["v"].shape, dtype=torch.float32, device="cuda")
    pool = d["pool"].clone()
    plan = gdn.PrefillPlan(d["q"], d["v"], out, case.n_seqs, state=pool)
    plan.prepare(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"])
    plan.scan(d["pool"], pool, out, d["slot_in"], d["slot_out"])
    torch.cuda.synchronize()
    return out, pool


def test_long_prefill_runs_in_cache_sized_ranges():
    """A long single sequence (129 chunks, weak decay so the state carried
    from range to range matters) runs as several chunk ranges inside one
    call: parity on sampled heads, and bitwise equal to the split-phase
    calls, which run the whole batch as one range."""
    case = gi.make_case("ranges_T8229", [8229], dtype="bf16", seed=91, decay="weak",
                        **gi.QWEN3_NEXT_HEADS)
    d = dev_case(case)
    out, pool = gpu_prefill(case, d=d, inplace=False)
    o1, p1 = _split_phase(case, d)
    assert torch.equal(out, o1) and torch.equal(pool, p1)
    ref_o, ref_s = oracle_case(case, heads=[0, 5, 16, 31])
    compare_prefill(case, out, pool, ref_o, ref_s, heads=[0, 5, 16, 31])


def test_long_prefill_f32_runs_in_ranges():
    """fp32 inputs (fp32 operands, larger factors: 3.5 MiB per chunk at these
    heads) over 71 chunks, which run as ranges of 32 chunks: parity on
    sampled heads and bitwise equal to the split-phase calls (one range)."""
    case = gi.make_case("ranges_f32_T4500", [4500], dtype="f32", seed=94, decay="weak",
                        **gi.QWEN3_NEXT_HEADS)
    d = dev_case(case)
    out, pool = gpu_prefill(case, d=d, inplace=False)
    o1, p1 = _split_phase(case, d)
    assert torch.equal(out, o1) and torch.equal(pool, p1)
    heads = [0, 7, 31]
    ref_o, ref_s = oracle_case(case, heads=heads)
    compare_prefill(case, out, pool, ref_o, ref_s, heads=heads)


@pytest.mark.parametrize("dtype,dk,dv,lens", [("bf16", 128, 128, [700, 129]), ("f32", 64, 64, [200, 1])])
def test_prefill_reads_no_workspace_byte_before_writing_it(dtype, dk, dv, lens):
    """The same call with a workspace filled with 0xff bytes (NaN as fp32
    and bf16) and with a zeroed one gives bitwise equal results: every byte
    the scan reads was written by the preparation of the same call.  The
    preparation leaves out the P fragments that lie wholly above the
    diagonal, which the scan reads through a range that ends before them."""
    import gated_deltanet_rule_amd as gdn
    case = gi.make_case(f"ws_dirty_{dtype}_{dk}", lens, 2, 4, dk, dv, dtype, seed=71, decay="weak",
                        n_slots=4, scatter_slots=True)
    d = dev_case(case)
    T = case.total_tokens
    dims = gdn._dims_from(d["q"], d["v"], torch.empty(d["v"].shape, device="meta"), 0.0, 1e-6,
                          d["pool"])
    need = gdn.chunked_workspace_size(dims, case.n_seqs, T)
    say(f"prefill {case.name}: lengths {lens}, workspace {need} bytes")

    def run(fill):
        ws = torch.full((need,), fill, dtype=torch.uint8, device="cuda")
        out = torch.empty(d["v"].shape, dtype=torch.float32, device="cuda")
        pool = d["pool"].clone()
        gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], pool, out, d["cu"],
                    d["slot_in"], d["slot_out"], ws)
        torch.cuda.synchronize()
        return out, pool

    o1, p1 = run(0)
    o2, p2 = run(255)
    assert torch.isfinite(o1).all() and torch.isfinite(p1).all()
    assert torch.equal(o1, o2) and torch.equal(p1, p2)


def test_one_range_workspace():
    """gdn_chunked_prefill with exactly gdn_chunked_prefill_workspace_size
    bytes (the factor slots of one 64-chunk range for 130 chunks) gives the
    results of the split-phase layout's full-size workspace bit for bit, with
    the workspace past that size untouched; 256 bytes less is rejected with
    GDN_ERR_WORKSPACE before anything is enqueued (outputs untouched)."""
    import gated_deltanet_rule_amd as gdn
    case = gi.make_case("ranges_ws_T8229", [8229], dtype="bf16", seed=95, decay="weak",
                        **gi.QWEN3_NEXT_HEADS)
    d = dev_case(case)
    T = case.total_tokens
    dims = gdn._dims_from(d["q"], d["v"], torch.empty(d["v"].shape, device="meta"), 0.0, 1e-6,
                          d["pool"])
    small = gdn.chunked_workspace_size(dims, 1, T)
    full = gdn.workspace_size(dims, 1, T)
    assert small < full
    say(f"workspace: {small} bytes for the call, {full} for the split-phase calls")

    def run(ws):
        out = torch.full(d["v"].shape, 7.0, dtype=torch.float32, device="cuda")
        pool = d["pool"].clone()
        gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], pool, out, d["cu"],
                    d["slot_in"], d["slot_out"], ws)
        torch.cuda.synchronize()
        return out, pool

    ws_full = torch.zeros(full, dtype=torch.uint8, device="cuda")
    o1, p1 = run(ws_full)
    ws_small = torch.zeros(full, dtype=torch.uint8, device="cuda")
    o2, p2 = run(ws_small[:small])
    assert torch.equal(o1, o2) and torch.equal(p1, p2)
    assert not ws_small[small:].any()
    out = torch.full(d["v"].shape, 7.0, dtype=torch.float32, device="cuda")
    pool = d["pool"].clone()
    with pytest.raises(gdn.GdnError) as e:
        gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], pool, out, d["cu"],
                    d["slot_in"], d["slot_out"], ws_small[:small - 256])
    assert e.value.status == 3     # GDN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (out == 7.0).all() and torch.equal(pool, d["pool"])


def test_varlen_sequences_across_range_boundaries():
    """Sequences that start and end inside ranges, end and start on a range
    boundary, span three ranges (9000 tokens), are empty or a single token,
    with the zero-state slot and scattered slots (ranges of 64 chunks at
    these heads)."""
    lengths = [1900, 0, 1, 2100, 64 * 33, 7, 9000, 3000, 65]
    case = gi.make_case("ranges_varlen", lengths, dtype="bf16", seed=92, decay="weak",
                        n_slots=20, scatter_slots=True, **gi.QWEN3_NEXT_HEADS)
    case.slot_in[3] = -1
    d = dev_case(case)
    out, pool = gpu_prefill(case, d=d, inplace=False)
    o1, p1 = _split_phase(case, d)
    assert torch.equal(out, o1) and torch.equal(pool, p1)
    heads = [0, 9, 22, 31]
    ref_o, ref_s = oracle_case(case, heads=heads)
    compare_prefill(case, out, pool, ref_o, ref_s, heads=heads)


@pytest.mark.parametrize("n_seqs", [1500, 5000])
def test_many_sequences(n_seqs):
    """Thousands of short ragged sequences in one call (empty ones included):
    the chunk table's loop over 1024-sequence blocks, and above 4096
    sequences its direct write of the descriptors."""
    rng = np.random.default_rng(n_seqs)
    lengths = [int(x) for x in rng.choice([0, 1, 2, 3, 17, 64, 65, 130], size=n_seqs)]
    case = gi.make_case(f"many_{n_seqs}", lengths, 1, 2, 32, 32, "bf16", seed=n_seqs + 1,
                        decay="weak", n_slots=n_seqs, scatter_slots=True)
    _check(case)


def test_single_call_65536_tokens():
    """The long-context workload as one call: 1024 chunks in 16 chunk ranges
    (every head)."""
    case = gi.make_case("one_call_65536", [65536], dtype="bf16", seed=93, decay="weak",
                        **gi.QWEN3_NEXT_HEADS)
    _check(case)


def test_f32_inputs_bf16_output():
    """fp32 inputs (fp32 matrix-core operands) with a bf16 output: the output
    is rounded once from fp32, held to 1e-4 rms + 2^-8 |ref|."""
    case = gi.make_case("f32_in_bf16_out", [1, 63, 64, 65, 200, 0], 2, 4, 64, 32, "f32", seed=94,
                        decay="weak", n_slots=8, scatter_slots=True)
    _check(case, out_dtype=torch.bfloat16)


@pytest.mark.parametrize("decay", ["zero", "weak"])
def test_bf16_state_carry_over_65536_tokens(decay):
    """bf16 inputs, no decay (g = 0) or weak decay, 65536 tokens fed as 128
    calls of 512 with the state carried in place, all 32 value heads: the
    state carried through 1024 chunks must not drift from the sequential
    recurrence.  Reports the output error per window of 128 chunks and the
    carried state's error after 8, 64, 256 and 1024 chunks (oracle runs on
    those prefixes)."""
    import gated_deltanet_rule_amd as gdn
    T, U = 65536, 512
    case = gi.make_case(f"carry_{decay}_T65536", [T], dtype="bf16", seed=97, decay=decay,
                        **gi.QWEN3_NEXT_HEADS)
    d = dev_case(case)
    out = torch.empty(d["v"].shape, dtype=torch.float32, device="cuda")
    pool = d["pool"].clone()
    snaps = {}
    for c, s0 in enumerate(range(0, T, U)):
        cu = torch.tensor([0, U], dtype=torch.int32, device="cuda")
        sl_in = d["slot_in"] if s0 == 0 else d["slot_out"]
        gdn.prefill(d["q"][s0:s0 + U], d["k"][s0:s0 + U], d["v"][s0:s0 + U], d["g"][s0:s0 + U],
                    d["beta"][s0:s0 + U], pool, pool, out[s0:s0 + U], cu, sl_in, d["slot_out"])
        if (c + 1) * U in (U, 8 * U, 32 * U, 128 * U):
            snaps[(c + 1) * U] = pool[int(case.slot_out[0])].clone()
    torch.cuda.synchronize()
    ref_o, ref_s = oracle_case(case)
    o = out.cpu().numpy().astype(np.float64)
    rms = float(np.sqrt(np.mean(ref_o ** 2)))
    assert np.all(np.isfinite(o))
    worst = 0.0
    for w0 in range(0, T, 128 * 64):
        e = float(np.max(np.abs(o[w0:w0 + 8192] - ref_o[w0:w0 + 8192]))) / rms
        say(f"  chunks [{w0 // 64}, {w0 // 64 + 128}): out err/rms {e:.3e}")
        worst = max(worst, e)
    assert worst <= TOL["bf16"]
    s0 = np.stack([case.pool[case.slot_in[0]]]).astype(np.float64)
    for n, snap in sorted(snaps.items()):
        if n == T:
            ref = ref_s[0]
        else:
            _, rs = oracle.run(case.q[:n], case.k[:n], case.v[:n], case.g[:n], case.beta[:n],
                               np.array([0, n], np.int32), s0)
            ref = rs[0]
        es, _ = rel_err(snap.cpu().numpy().astype(np.float64), ref)
        say(f"  state after {n // 64} chunks: err/rms {es:.3e}")
        assert es <= TOL["bf16"]
