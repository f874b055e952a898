"""gdn_chunked_prefill_noalloc (the allocation-free entry point, for callers
that cannot allocate device memory) through the C ABI against
gdn_chunked_prefill on the same inputs: two calls in a row on one GPU, the
second with a smaller input, each bitwise equal to the workspace entry
point (and the first also within the bf16 tolerance of the fp64 oracle);
then a batch that does not fit the library's scratch is rejected before
anything runs."""
import numpy as np
import pytest
import torch

import workloads as gi
from gpu_harness import TOL, compare_prefill, dev_case, oracle_case, say

pytestmark = pytest.mark.gpu


def _both(case):
    import gated_deltanet_rule_amd as gdn
    d = dev_case(case)
    outs = []
    for fn in (gdn.prefill, gdn.prefill_noalloc):
        out = torch.full(d["v"].shape, float("nan"), dtype=torch.float32, device="cuda")
        pool = d["pool"].clone()
        fn(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], pool, out, d["cu"], d["slot_in"],
           d["slot_out"])
        torch.cuda.synchronize()
        outs.append((out, pool))
    (o1, p1), (o2, p2) = outs
    assert torch.equal(o1, o2), "output differs from gdn_chunked_prefill"
    assert torch.equal(p1, p2), "state pool differs from gdn_chunked_prefill"
    return o2, p2


def test_noalloc_matches_the_workspace_entry_point_twice():
    # 1. the 4096-token prefill with Qwen3-Next heads: its factors outgrow the
    #    scratch, so it runs as several shorter chunk ranges
    case = gi.config1()
    say(f"noalloc call 1: {case.name}")
    o, p = _both(case)
    heads = [0, 13, 31]
    ref_o, ref_s = oracle_case(case, heads=heads)
    compare_prefill(case, o, p, ref_o, ref_s, heads=heads, tol=TOL["bf16"])
    # 2. a smaller ragged batch right after, on the same scratch
    small = gi.make_case("noalloc_small", [17, 64, 65, 130, 0, 1], 2, 4, 64, 64, "bf16", seed=111,
                         decay="weak", n_slots=9, scatter_slots=True)
    say(f"noalloc call 2: {small.name}")
    o, p = _both(small)
    ref_o, ref_s = oracle_case(small)
    compare_prefill(small, o, p, ref_o, ref_s, tol=TOL["bf16"])


def test_noalloc_rejects_a_batch_beyond_its_scratch():
    """The epilogue with a bf16 out stages 4*T*H_v*d_v bytes of fp32 output:
    8192 tokens at Qwen3-Next heads need 128 MiB, more than the scratch."""
    import gated_deltanet_rule_amd as gdn
    H = gi.QWEN3_NEXT_HEADS
    T = 8192
    dev = "cuda"
    q = torch.zeros(T, H["H_k"], H["d_k"], dtype=torch.bfloat16, device=dev)
    v = torch.zeros(T, H["H_v"], H["d_v"], dtype=torch.bfloat16, device=dev)
    g = torch.zeros(T, H["H_v"], dtype=torch.float32, device=dev)
    pool = torch.zeros(1, H["H_v"], H["d_k"], H["d_v"], dtype=torch.float32, device=dev)
    out = torch.full((T, H["H_v"], H["d_v"]), 3.0, dtype=torch.bfloat16, device=dev)
    z = torch.zeros_like(v)
    nw = torch.ones(H["d_v"], dtype=torch.float32, device=dev)
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    sl = torch.zeros(1, dtype=torch.int32, device=dev)
    with pytest.raises(gdn.GdnError) as e:
        gdn.prefill_noalloc(q, q, v, g, g, pool, pool, out, cu, sl, sl, z=z, norm_w=nw)
    torch.cuda.synchronize()
    assert e.value.status == 3 and "scratch" in str(e.value)
    assert bool((out == 3.0).all())
