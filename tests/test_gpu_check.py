"""GDN_CHECK=1: device-side preconditions (cu_seqlens, slot lists) are
validated before any kernel of the call runs; a bad call returns
GDN_ERR_INVALID_ARG and leaves every output untouched, a good one gives the
same results as an unchecked call."""
import os

import numpy as np
import pytest
import torch

import workloads as gi
from gpu_harness import dev_case, gpu_prefill

pytestmark = pytest.mark.gpu

INVALID = 1


@pytest.fixture
def check_mode():
    old = os.environ.get("GDN_CHECK")
    os.environ["GDN_CHECK"] = "1"
    yield
    if old is None:
        del os.environ["GDN_CHECK"]
    else:
        os.environ["GDN_CHECK"] = old


def _varlen():
    case = gi.make_case("check_varlen", [17, 64, 65, 130], 2, 4, 64, 64, "bf16", seed=101,
                        n_slots=8, scatter_slots=True)
    return case, dev_case(case)


def _prefill(gdn, d, cu, slot_in, slot_out, out, pool_out):
    gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], pool_out, out, cu,
                slot_in, slot_out)


def test_valid_calls_pass_and_match(check_mode):
    case, d = _varlen()
    out_c, pool_c = gpu_prefill(case, d=d, inplace=False)
    del os.environ["GDN_CHECK"]
    out_u, pool_u = gpu_prefill(case, d=d, inplace=False)
    os.environ["GDN_CHECK"] = "1"
    assert torch.equal(out_c, out_u) and torch.equal(pool_c, pool_u)


@pytest.mark.parametrize("bad", ["start", "order", "end"])
def test_prefill_rejects_bad_cu_seqlens(check_mode, bad):
    import gated_deltanet_rule_amd as gdn
    case, d = _varlen()
    cu = case.cu_seqlens.copy()
    if bad == "start":
        cu[0] = 1
    elif bad == "order":
        cu[2], cu[3] = cu[3], cu[2]
    else:
        cu[-1] -= 1
    cu_d = torch.from_numpy(cu).cuda()
    out = torch.full(d["v"].shape, float("nan"), device="cuda")
    pool_out = torch.full_like(d["pool"], float("nan"))
    with pytest.raises(gdn.GdnError) as e:
        _prefill(gdn, d, cu_d, d["slot_in"], d["slot_out"], out, pool_out)
    torch.cuda.synchronize()
    assert e.value.status == INVALID and "GDN_CHECK" in str(e.value)
    assert torch.isnan(out).all() and torch.isnan(pool_out).all()


@pytest.mark.parametrize("bad", ["dup", "alias"])
def test_prefill_rejects_bad_slots(check_mode, bad):
    import gated_deltanet_rule_amd as gdn
    case, d = _varlen()
    si, so = case.slot_in.copy(), case.slot_out.copy()
    if bad == "dup":
        so[3] = so[1]
    else:
        # sequence 2 writes a fresh slot, sequence 0 writes the slot 2 reads
        so[2] = next(x for x in range(case.pool.shape[0]) if x not in si and x not in so)
        so[0] = si[2]
    out = torch.full(d["v"].shape, float("nan"), device="cuda")
    pool_out = torch.full_like(d["pool"], float("nan"))
    with pytest.raises(gdn.GdnError) as e:
        _prefill(gdn, d, d["cu"], torch.from_numpy(si).cuda(), torch.from_numpy(so).cuda(), out, pool_out)
    torch.cuda.synchronize()
    assert e.value.status == INVALID
    assert ("same slot" in str(e.value)) == (bad == "dup")
    assert torch.isnan(out).all()


def test_decode_and_multi_token_checks(check_mode):
    import gated_deltanet_rule_amd as gdn
    dc = gi.make_decode("check_decode", 6, 2, 2, 4, 64, 64, "bf16", seed=102)
    f = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(t)
    dt = torch.bfloat16
    q, k, v = f(dc.q[0], dt), f(dc.k[0], dt), f(dc.v[0], dt)
    g, b, pool = f(dc.g[0]), f(dc.beta[0]), f(dc.pool)
    slots = dc.slots.copy()
    out = torch.empty(v.shape, device="cuda")
    gdn.decode_step(q, k, v, g, b, pool, pool.clone(), out, f(slots, torch.int32), f(slots, torch.int32))
    bad = slots.copy()
    bad[4] = bad[0]
    with pytest.raises(gdn.GdnError) as e:
        gdn.decode_step(q, k, v, g, b, pool, pool.clone(), out, f(slots, torch.int32), f(bad, torch.int32))
    assert e.value.status == INVALID
    # multi-token: 6 sequences of 1 token each, then a decreasing cu_seqlens
    cu = np.arange(7, dtype=np.int32)
    gdn.decode_multi(q, k, v, g, b, pool, pool.clone(), out, f(cu, torch.int32), f(slots, torch.int32),
                     f(slots, torch.int32))
    cu_bad = cu.copy()
    cu_bad[3] = 5
    with pytest.raises(gdn.GdnError) as e:
        gdn.decode_multi(q, k, v, g, b, pool, pool.clone(), out, f(cu_bad, torch.int32),
                         f(slots, torch.int32), f(slots, torch.int32))
    assert e.value.status == INVALID
    torch.cuda.synchronize()


def test_split_phase_checks(check_mode):
    import gated_deltanet_rule_amd as gdn
    case, d = _varlen()
    out = torch.empty(d["v"].shape, device="cuda")
    pool = d["pool"].clone()
    plan = gdn.PrefillPlan(d["q"], d["v"], out, case.n_seqs, state=pool)
    cu = case.cu_seqlens.copy()
    cu[-1] += 3
    with pytest.raises(gdn.GdnError):
        plan.prepare(d["q"], d["k"], d["v"], d["g"], d["beta"], torch.from_numpy(cu).cuda())
    plan.prepare(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"])
    so = case.slot_out.copy()
    so[2] = so[0]
    with pytest.raises(gdn.GdnError):
        plan.scan(d["pool"], pool, out, d["slot_in"], torch.from_numpy(so).cuda())
    plan.scan(d["pool"], pool, out, d["slot_in"], d["slot_out"])
    torch.cuda.synchronize()


def test_slot_indices_checked_against_the_pool_size(check_mode):
    """With the pool size known (dims.n_slots, which the binding takes from
    the pools), a slot index at or past it is rejected on every entry point
    before anything runs; negative indices (zero state / state not stored)
    stay valid, and so does the last slot."""
    import gated_deltanet_rule_amd as gdn
    case, d = _varlen()
    n = case.pool.shape[0]
    si, so = case.slot_in.copy(), case.slot_out.copy()
    for which, idx in (("in", n), ("out", n), ("out", n + 1000)):
        bi, bo = si.copy(), so.copy()
        (bi if which == "in" else bo)[1] = idx
        out = torch.full(d["v"].shape, float("nan"), device="cuda")
        pool_out = torch.full_like(d["pool"], float("nan"))
        with pytest.raises(gdn.GdnError) as e:
            _prefill(gdn, d, d["cu"], torch.from_numpy(bi).cuda(), torch.from_numpy(bo).cuda(),
                     out, pool_out)
        torch.cuda.synchronize()
        assert e.value.status == INVALID and "n_slots" in str(e.value)
        assert torch.isnan(out).all() and torch.isnan(pool_out).all()
    # the last slot and negative indices are valid
    bi, bo = si.copy(), so.copy()
    free = [x for x in range(n) if x not in si and x not in so]
    bo[0] = n - 1 if n - 1 in free else bo[0]
    bi[2] = -1
    out = torch.empty(d["v"].shape, device="cuda")
    _prefill(gdn, d, d["cu"], torch.from_numpy(bi).cuda(), torch.from_numpy(bo).cuda(), out,
             d["pool"].clone())
    torch.cuda.synchronize()
    # decode and multi-token decode
    dc = gi.make_decode("check_range", 4, 1, 2, 4, 64, 64, "bf16", seed=103, n_slots=6)
    f = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(t)
    q, k, v = f(dc.q[0], torch.bfloat16), f(dc.k[0], torch.bfloat16), f(dc.v[0], torch.bfloat16)
    g, b, pool = f(dc.g[0]), f(dc.beta[0]), f(dc.pool)
    out = torch.empty(v.shape, device="cuda")
    bad = np.array([0, 1, 6, 3], np.int32)
    with pytest.raises(gdn.GdnError) as e:
        gdn.decode_step(q, k, v, g, b, pool, pool.clone(), out, f(bad, torch.int32), f(bad, torch.int32))
    assert e.value.status == INVALID
    with pytest.raises(gdn.GdnError) as e:
        gdn.decode_multi(q, k, v, g, b, pool, pool.clone(), out, f(np.arange(5, dtype=np.int32), torch.int32),
                         f(bad, torch.int32), f(bad, torch.int32))
    assert e.value.status == INVALID
    ok = np.array([0, 1, 5, 3], np.int32)
    gdn.decode_step(q, k, v, g, b, pool, pool.clone(), out, f(ok, torch.int32), f(ok, torch.int32))
    torch.cuda.synchronize()


def test_concurrent_checked_calls_keep_their_own_verdicts(check_mode):
    """Checked calls from several host threads at once, each on its own
    stream, half of them invalid (duplicate output slots): every call gets its
    own verdict (the result word is per call)."""
    import threading
    import gated_deltanet_rule_amd as gdn
    case, d = _varlen()
    so_bad = case.slot_out.copy()
    so_bad[3] = so_bad[1]
    good_so, bad_so = d["slot_out"], torch.from_numpy(so_bad).cuda()
    results = {}

    def worker(i):
        s = torch.cuda.Stream()
        outs = []
        for r in range(6):
            bad = (i + r) % 2 == 1
            out = torch.empty(d["v"].shape, device="cuda")
            pool_out = d["pool"].clone()
            try:
                with torch.cuda.stream(s):
                    gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], pool_out, out,
                                d["cu"], d["slot_in"], bad_so if bad else good_so, stream=s)
                outs.append((bad, None))
            except gdn.GdnError as e:
                outs.append((bad, e.status))
        s.synchronize()
        results[i] = outs

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert len(results) == 4
    for i, outs in results.items():
        for bad, status in outs:
            assert status == (INVALID if bad else None), (i, bad, status)
