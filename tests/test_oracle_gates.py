"""Pins of the oracle's gate activations (no GPU).

The layer turns its raw projections into the operator's inputs as the page
"Optimization: Qwen3 next autoregressive pass (#17996)" builds them in
build_layer_attn_linear: beta = sigmoid(b); gate = softplus(a + ssm_dt) *
ssm_a, with ssm_dt and ssm_a per value head.  The pins below check
``oracle.gates`` against hand-worked values, identities of softplus and
sigmoid, element-by-element evaluation with the textbook ``math`` routines,
and the extremes, and show that plausible mistakes (a dropped bias, a wrong
sign, swapped per-head parameters, the rate applied twice, a logistic in place
of softplus) are caught."""
import math

import numpy as np
import pytest

import oracle


def _pins(gates, softplus, sigmoid):
    """Returns a list of (name, passed) for one implementation."""
    out = []
    # hand-worked: softplus(0) = ln 2, sigmoid(ln 3) = 3/4
    g, b = gates(np.array([[0.25]]), np.array([[math.log(3.0)]]), np.array([-2.0]), np.array([-0.25]))
    out.append(("hand_value_g", abs(g[0, 0] - (-2.0 * math.log(2.0))) < 1e-15))
    out.append(("hand_value_beta", abs(b[0, 0] - 0.75) < 1e-15))
    # identities
    x = np.linspace(-30, 30, 241)
    out.append(("softplus_odd_part", np.allclose(softplus(x) - softplus(-x), x, rtol=0, atol=1e-12)))
    out.append(("sigmoid_symmetry", np.allclose(sigmoid(x) + sigmoid(-x), 1.0, rtol=0, atol=1e-15)))
    h = 1e-6
    xs = np.linspace(-6, 6, 49)
    der = (softplus(xs + h) - softplus(xs - h)) / (2 * h)
    out.append(("softplus_derivative_is_sigmoid", np.allclose(der, sigmoid(xs), rtol=0, atol=1e-8)))
    # element by element against math.log1p / math.exp, distinct per-head parameters
    rng = np.random.default_rng(5)
    T, H = 7, 5
    a = rng.standard_normal((T, H)) * 3
    bb = rng.standard_normal((T, H)) * 3
    sa = -rng.uniform(0.5, 8.0, H)
    sd = rng.uniform(-1.0, 1.0, H)
    G, B = gates(a, bb, sa, sd)
    ok_g = ok_b = True
    for t in range(T):
        for hh in range(H):
            y = a[t, hh] + sd[hh]
            ref_g = math.log1p(math.exp(y)) * sa[hh]
            ref_b = 1.0 / (1.0 + math.exp(-bb[t, hh]))
            ok_g &= abs(G[t, hh] - ref_g) <= 1e-14 * max(1.0, abs(ref_g))
            ok_b &= abs(B[t, hh] - ref_b) <= 1e-15
    out.append(("elementwise_g", bool(ok_g)))
    out.append(("elementwise_beta", bool(ok_b)))
    # sign and extremes (no overflow, correct limits)
    out.append(("g_nonpositive", bool(np.all(G <= 0))))
    big = np.array([[800.0, -800.0]])
    gg, bb2 = gates(big, big, np.array([-1.0, -1.0]), np.array([0.0, 0.0]))
    out.append(("extremes", bool(np.isfinite(gg).all() and gg[0, 0] == -800.0 and gg[0, 1] <= 0
                                 and bb2[0, 0] == 1.0 and bb2[0, 1] == 0.0)))
    return out


def test_oracle_gates_pass_every_pin():
    res = _pins(oracle.gates, oracle.softplus, oracle.sigmoid)
    bad = [n for n, ok in res if not ok]
    assert not bad, bad


def _mutant(kind):
    sp, sg = oracle.softplus, oracle.sigmoid

    def gates(a, b, ssm_a, ssm_dt):
        a = np.asarray(a, np.float64)
        sa = np.asarray(ssm_a, np.float64)[None, :]
        sd = np.asarray(ssm_dt, np.float64)[None, :]
        if kind == "no_bias":
            return sp(a) * sa, sg(b)
        if kind == "bias_sign":
            return sp(a - sd) * sa, sg(b)
        if kind == "swapped_params":
            return sp(a + sa) * sd, sg(b)
        if kind == "rate_exp":
            return sp(a + sd) * -np.exp(-sa), sg(b)
        if kind == "logistic_gate":
            return sg(a + sd) * sa, sg(b)
        if kind == "beta_softplus":
            return sp(a + sd) * sa, sp(b)
        raise ValueError(kind)
    return gates, sp, sg


@pytest.mark.parametrize("kind", ["no_bias", "bias_sign", "swapped_params", "rate_exp",
                                  "logistic_gate", "beta_softplus"])
def test_gate_mutation_is_caught(kind):
    res = _pins(*_mutant(kind))
    assert any(not ok for _, ok in res), f"mutation {kind} passed every pin"


def test_mutated_softplus_is_caught():
    bad_sp = lambda x: np.log(1.0 + np.exp(np.asarray(x, np.float64)))   # overflows at 800
    def gates(a, b, sa, sd):
        return bad_sp(np.asarray(a) + np.asarray(sd)[None, :]) * np.asarray(sa)[None, :], oracle.sigmoid(b)
    with np.errstate(over="ignore"):
        res = _pins(gates, bad_sp, oracle.sigmoid)
    assert any(not ok for _, ok in res)
