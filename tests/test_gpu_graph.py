"""The calls enqueue only kernels on the caller's stream (no allocation, no
memset, no synchronisation), so they can be captured into a HIP graph.  Each
graph is replayed several times with eager work and synchronisations in
between, and every replay is compared with the eager result."""
import numpy as np
import pytest
import torch

import workloads as gi
from gpu_harness import dev_case

pytestmark = pytest.mark.gpu


def _warm(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()


def test_prefill_graph_replays_match_eager():
    import gated_deltanet_rule_amd as gdn
    case = gi.make_case("graph_prefill", [300, 0, 77, 650], 2, 4, 128, 128, "bf16", seed=111,
                        decay="weak", n_slots=6, scatter_slots=True)
    d = dev_case(case)
    out = torch.empty(d["v"].shape, device="cuda")
    plan = gdn.PrefillPlan(d["q"], d["v"], out, case.n_seqs, state=d["pool"])
    ws = plan.workspace                     # caller-owned, sized by gdn_prefill_workspace_size
    pool_out = d["pool"].clone()

    def call():
        gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], pool_out, out, d["cu"],
                    d["slot_in"], d["slot_out"], ws)

    call()
    torch.cuda.synchronize()
    ref_out, ref_pool = out.clone(), pool_out.clone()
    _warm(call)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(4):
        out.fill_(float("nan"))
        pool_out.copy_(d["pool"])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(pool_out, ref_pool), f"replay {rep}"


def test_decode_graph_steps_match_eager_steps():
    import gated_deltanet_rule_amd as gdn
    dc = gi.make_decode("graph_decode", 16, 6, 2, 4, 128, 128, "bf16", seed=112)
    f = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(t)
    dt = torch.bfloat16
    q, k, v, g, b = (f(dc.q, dt), f(dc.k, dt), f(dc.v, dt), f(dc.g), f(dc.beta))
    slots = f(dc.slots, torch.int32)
    # eager: six steps in place
    pool_e = f(dc.pool)
    outs_e = torch.empty(v.shape, device="cuda")
    for s in range(dc.n_steps):
        gdn.decode_step(q[s], k[s], v[s], g[s], b[s], pool_e, pool_e, outs_e[s], slots, slots)
    torch.cuda.synchronize()
    # graph: one step reading static inputs, replayed once per step
    pool_g = f(dc.pool)
    sq, sk, sv, sg, sb = q[0].clone(), k[0].clone(), v[0].clone(), g[0].clone(), b[0].clone()
    sout = torch.empty(v[0].shape, device="cuda")

    def step():
        gdn.decode_step(sq, sk, sv, sg, sb, pool_g, pool_g, sout, slots, slots)

    warm_pool = pool_g.clone()
    _warm(step)
    pool_g.copy_(warm_pool)                  # the warm-up step is undone
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    pool_g.copy_(warm_pool)                  # capture does not run the step, but be explicit
    torch.cuda.synchronize()
    for s in range(dc.n_steps):
        sq.copy_(q[s]); sk.copy_(k[s]); sv.copy_(v[s]); sg.copy_(g[s]); sb.copy_(b[s])
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(sout, outs_e[s]), f"step {s}"
    assert torch.equal(pool_g, pool_e)
