"""Seeded input generators: determinism, dtype rounding, recipe shapes (no GPU)."""
import hashlib

import numpy as np
import torch

import gdn_inputs as gi
import oracle
import workloads


def _h(*arrs):
    m = hashlib.sha256()
    for a in arrs:
        m.update(np.ascontiguousarray(a).tobytes())
    return m.hexdigest()


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -2.00781250, 0.0, -0.0], np.float32)])
    ours = gi.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_generators_are_deterministic():
    a, b = gi.config0(), gi.config0()
    assert _h(a.q, a.k, a.v, a.g, a.beta, a.pool) == _h(b.q, b.k, b.v, b.g, b.beta, b.pool)
    c = gi.make_case("x", [5, 9], 2, 4, 16, 16, "bf16", seed=7, n_slots=8, scatter_slots=True)
    d = gi.make_case("x", [5, 9], 2, 4, 16, 16, "bf16", seed=7, n_slots=8, scatter_slots=True)
    assert _h(c.q, c.v, c.pool, c.slot_in) == _h(d.q, d.v, d.pool, d.slot_in)


def test_recipe_shapes_and_ranges():
    c = workloads.config0()
    assert c.q.shape == (128, 2, 32) and c.v.shape == (128, 2, 32)
    assert np.all(c.g <= 0) and np.all((c.beta > 0) & (c.beta < 1))
    assert not c.pool.any() and np.all(c.slot_in == -1)
    n = np.linalg.norm(c.q.astype(np.float64), axis=-1)
    assert np.allclose(n, 1.0, atol=1e-6)
    b = gi.make_case("b", [70], 2, 4, 32, 32, "bf16", seed=3)
    # bf16 storage: low 16 bits are zero
    assert not (b.q.view(np.uint32) & 0xFFFF).any()
    assert not (b.v.view(np.uint32) & 0xFFFF).any()
    # strong decay: ssm_a = -U(1, 16); no gate bias by default; raw projections per token-head
    assert np.all(b.ssm_a <= -1) and np.all(b.ssm_a >= -16)
    assert not b.ssm_dt.any()
    assert b.raw_a.shape == (70, 4) and b.raw_b.shape == (70, 4)
    assert b.g is None and b.beta is None      # the generator evaluates no activation
    bb = gi.make_case("b", [70], 2, 4, 32, 32, "bf16", seed=3, gate_bias=True)
    assert np.all(np.abs(bb.ssm_dt) <= 1) and bb.ssm_dt.any()
    w = gi.make_case("w", [70], 2, 4, 32, 32, "bf16", seed=3, decay="weak")
    assert np.all(w.ssm_a <= -0.001) and np.all(w.ssm_a >= -0.01)


def test_decode_repacking():
    dc = workloads.make_decode("d", 3, 5, 1, 2, 8, 8, "f32", seed=1)
    q, k, v, g, beta, cu = gi.decode_as_sequences(dc)
    assert list(cu) == [0, 5, 10, 15]
    assert np.array_equal(q[5 + 2], dc.q[2, 1]) and np.array_equal(v[10 + 4], dc.v[4, 2])


def test_layer_inputs_recipe():
    a = gi.make_layer_inputs(33, 5, 2, 4, 32, 64, "bf16", seed=9)
    b = gi.make_layer_inputs(33, 5, 2, 4, 32, 64, "bf16", seed=9)
    C = gi.conv_dim(2, 4, 32, 64)
    assert C == 2 * 2 * 32 + 4 * 64
    assert a.qkv.shape == (33, C) and a.conv_w.shape == (C, gi.D_CONV)
    assert a.conv_pool.shape == (5, C, gi.D_CONV - 1) and a.z.shape == (33, 4, 64)
    assert a.norm_w.shape == (64,)
    for f in ("qkv", "conv_w", "conv_pool", "z", "norm_w"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    # bf16 storage: values survive a bf16 round trip unchanged
    for f in ("qkv", "conv_pool", "z"):
        x = getattr(a, f)
        assert np.array_equal(gi.round_to_bf16(x), x), f
    # a stream of its own: the operator inputs of the same seed are unchanged
    c1 = gi.make_case("x", [33], 2, 4, 32, 64, "bf16", seed=9)
    c2 = gi.make_case("x", [33], 2, 4, 32, 64, "bf16", seed=9)
    assert np.array_equal(c1.q, c2.q)
    assert abs(float(np.std(a.qkv)) - 1.0) < 0.05


def test_workload_gate_recipe():
    """The workloads' gates: beta = sigmoid(N(0,1)), g = -exp(A_log) softplus(N(0,1))
    with A_log = log U(1,16): the harness applies the activations to the
    generator's raw draws (ssm_dt = 0), and the draws have the stated laws."""
    c = workloads.config1(T=2048)
    assert not c.ssm_dt.any()
    g, beta = oracle.gates(c.raw_a, c.raw_b, c.ssm_a, c.ssm_dt)
    assert np.array_equal(c.g, g.astype(np.float32))
    assert np.array_equal(c.beta, beta.astype(np.float32))
    # raw draws: standard normal
    for x in (c.raw_a, c.raw_b):
        assert abs(float(np.mean(x))) < 0.01 and abs(float(np.std(x)) - 1.0) < 0.01
    # E[sigmoid(N(0,1))] = 1/2; E[softplus(N(0,1))] = 0.8063...
    assert abs(float(np.mean(c.beta)) - 0.5) < 0.01
    sp = c.g / c.ssm_a[None, :]
    assert abs(float(np.mean(sp)) - 0.8063) < 0.01
    # decay rate -exp(log U(1, 16)) per head
    assert np.all((-c.ssm_a >= 1) & (-c.ssm_a <= 16))
    # the decode workload uses the same recipe
    d = workloads.config2(n_steps=4)
    g2, b2 = oracle.gates(d.raw_a.reshape(-1, 32), d.raw_b.reshape(-1, 32), d.ssm_a, d.ssm_dt)
    assert np.array_equal(d.g.reshape(-1, 32), g2.astype(np.float32))
    assert np.array_equal(d.beta.reshape(-1, 32), b2.astype(np.float32))
