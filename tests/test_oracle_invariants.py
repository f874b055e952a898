"""Structural properties of the operator checked on the fp64 oracle (no GPU).

These follow from the definition (per-(sequence, head) independence, the
slot/state carry of "ik_llama.cpp src/llama-delta-net.cpp"
build_layer_attn_linear_core, the GQA repeat of the same function, and the
algebra of the recurrence) rather than from any implementation.
"""
import numpy as np
import pytest

import oracle
from pins import _rand_inputs, _rel

TOL = 1e-10


@pytest.fixture(scope="module")
def data():
    rng = np.random.default_rng(21)
    return _rand_inputs(rng, [23, 70, 1, 0, 41], 2, 4, 16, 16, decay=(0.01, 0.3))


def test_varlen_packing_equals_separate_runs(data):
    q, k, v, g, b, cu, s0 = data
    out, sf = oracle.recurrent(q, k, v, g, b, cu, s0)
    for s in range(len(cu) - 1):
        a, e = cu[s], cu[s + 1]
        o1, s1 = oracle.recurrent(q[a:e], k[a:e], v[a:e], g[a:e], b[a:e],
                                  np.array([0, e - a]), s0[s:s + 1])
        if e > a:
            assert _rel(o1, out[a:e]) < TOL
        assert _rel(s1[0], sf[s]) < TOL


def test_zero_length_sequence_passes_state_through(data):
    q, k, v, g, b, cu, s0 = data
    _, sf = oracle.recurrent(q, k, v, g, b, cu, s0)
    assert cu[3] == cu[4]
    assert np.array_equal(sf[3], s0[3])


def test_state_carry_across_calls_equals_one_call(data):
    """ubatch split: tokens [0, m) then [m, T) with the state carried."""
    q, k, v, g, b, cu, s0 = data
    a, e = cu[1], cu[2]
    full_o, full_s = oracle.recurrent(q[a:e], k[a:e], v[a:e], g[a:e], b[a:e],
                                      np.array([0, e - a]), s0[1:2])
    for m in (1, 17, 64, 69):
        o1, s1 = oracle.recurrent(q[a:a + m], k[a:a + m], v[a:a + m], g[a:a + m],
                                  b[a:a + m], np.array([0, m]), s0[1:2])
        o2, s2 = oracle.recurrent(q[a + m:e], k[a + m:e], v[a + m:e], g[a + m:e],
                                  b[a + m:e], np.array([0, e - a - m]), s1)
        assert _rel(np.concatenate([o1, o2]), full_o) < TOL
        assert _rel(s2, full_s) < TOL


def test_gqa_equals_explicit_duplication(data):
    """H_v/H_k = 2 with blocked sharing == H_k = H_v with each key head repeated."""
    q, k, v, g, b, cu, s0 = data
    out, sf = oracle.recurrent(q, k, v, g, b, cu, s0)
    qd = np.repeat(q, 2, axis=1)   # key head j -> value heads 2j, 2j+1
    kd = np.repeat(k, 2, axis=1)
    o2, s2 = oracle.recurrent(qd, kd, v, g, b, cu, s0)
    assert _rel(o2, out) < 1e-14 and _rel(s2, sf) < 1e-14


def test_affine_in_initial_state(data):
    q, k, v, g, b, cu, s0 = data
    rng = np.random.default_rng(5)
    s1 = rng.standard_normal(s0.shape)
    o0, f0 = oracle.recurrent(q, k, v, g, b, cu, None)
    oa, fa = oracle.recurrent(q, k, v, g, b, cu, s0)
    ob, fb = oracle.recurrent(q, k, v, g, b, cu, s1)
    oc, fc = oracle.recurrent(q, k, v, g, b, cu, 0.3 * s0 + 0.7 * s1)
    assert _rel(oc, 0.3 * oa + 0.7 * ob) < TOL
    assert _rel(fc, 0.3 * fa + 0.7 * fb) < TOL
    # and the zero state is the affine offset
    od, fd = oracle.recurrent(q, k, v, g, b, cu, 2 * s0)
    assert _rel(od - oa, oa - o0) < 1e-8


def test_linear_in_values_with_zero_state(data):
    q, k, v, g, b, cu, _ = data
    rng = np.random.default_rng(6)
    v2 = rng.standard_normal(v.shape).astype(np.float32)
    o1, f1 = oracle.recurrent(q, k, v, g, b, cu, None)
    o2, f2 = oracle.recurrent(q, k, v2, g, b, cu, None)
    o3, f3 = oracle.recurrent(q, k, (v.astype(np.float64) + v2).astype(np.float32), g, b, cu, None)
    # v + v2 is rounded to fp32: compare against the fp32-rounded sum's linearity
    vs = (v.astype(np.float64) + v2).astype(np.float32).astype(np.float64)
    assert np.max(np.abs(vs - v - v2)) < 1e-6
    assert _rel(o3, o1 + o2) < 1e-6
    o4, _ = oracle.recurrent(q, k, 2 * v, g, b, cu, None)
    assert _rel(o4, 2 * o1) < 1e-14


def test_head_permutation_equivariance(data):
    """Permuting key heads (with their value-head groups) permutes the results."""
    q, k, v, g, b, cu, s0 = data
    out, sf = oracle.recurrent(q, k, v, g, b, cu, s0)
    kp = [1, 0]
    vp = [2, 3, 0, 1]
    o2, s2 = oracle.recurrent(q[:, kp], k[:, kp], v[:, vp], g[:, vp], b[:, vp], cu, s0[:, vp])
    assert np.array_equal(o2, out[:, vp]) and np.array_equal(s2, sf[:, vp])


def test_head_subset_and_thread_count(data):
    q, k, v, g, b, cu, s0 = data
    out, sf = oracle.recurrent(q, k, v, g, b, cu, s0, threads=1)
    o2, s2 = oracle.recurrent(q, k, v, g, b, cu, s0, threads=7)
    assert np.array_equal(out, o2) and np.array_equal(sf, s2)
    o3, s3 = oracle.recurrent(q, k, v, g, b, cu, s0, heads=[3, 1])
    assert np.array_equal(o3[:, [3, 1]], out[:, [3, 1]])
    assert np.array_equal(s3[:, [3, 1]], sf[:, [3, 1]])
    assert not o3[:, [0, 2]].any()


def test_strong_decay_stays_finite():
    """Chunk-level cumulative decays far below e^-87 (fp32 underflow) are fine."""
    rng = np.random.default_rng(22)
    q, k, v, g, b, cu, s0 = _rand_inputs(rng, [256], 1, 1, 16, 16, decay=(8.0, 16.0))
    assert np.sum(g[:64, 0]) < -200
    o, s = oracle.recurrent(q, k, v, g, b, cu, s0)
    oc, sc = oracle.chunked(q, k, v, g, b, cu, s0, chunk=64)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(oc))
    assert _rel(oc, o) < TOL and _rel(sc, s) < TOL
