"""Pins of the oracle's layer prologue and epilogue (no GPU).

``oracle.layer`` follows build_layer_attn_linear_core on the page
"ik_llama.cpp src/llama-delta-net.cpp": a short causal convolution with a
per-slot state and SiLU over the mixed q|k|v rows before the operator, and
the gated RMSNorm rms_norm(o) * w * silu(z) after it.  The pins check it
against hand-worked values, library routines on special cases
(numpy.convolve, torch's rms_norm and silu, math.exp), the T=1 closed form of
the operator through the whole layer, and structural facts (streaming the
rows in pieces with the carried state, packing sequences, state pass-through
for empty sequences).  Each plausible mistake planted in a copy of the oracle
(reversed taps, a reversed or ignored state, the wrong state kept, SiLU
missing or on the wrong operand, sum for mean, the epsilon dropped, the norm
over the wrong axis, q and k swapped) fails at least one pin."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import layer as L


def _silu_math(x):
    return np.vectorize(lambda t: t / (1.0 + math.exp(-t)))(np.asarray(x, np.float64))


# ---------------------------------------------------------------------------
# convolution + SiLU
# ---------------------------------------------------------------------------

def conv_pins(conv_silu):
    out = []
    # hand-worked: one channel, taps 1 2 3 4, state (0, 0, 1), rows 2, -1
    y, s = conv_silu(np.array([[2.0], [-1.0]]), np.array([[1.0, 2.0, 3.0, 4.0]]),
                     np.array([0, 2]), np.array([[[0.0, 0.0, 1.0]]]))
    out.append(("hand_values", np.allclose(y[:, 0], [11 / (1 + math.exp(-11)), 4 / (1 + math.exp(-4))],
                                           rtol=0, atol=1e-14)))
    out.append(("hand_state", np.array_equal(s[0, 0], [1.0, 2.0, -1.0])))
    rng = np.random.default_rng(11)
    T, C, d = 9, 5, 4
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, d))
    s0 = rng.standard_normal((1, C, d - 1))
    cu = np.array([0, T])
    y, s = conv_silu(x, w, cu, s0)
    # every channel against numpy.convolve on the state-extended rows
    ok = True
    for c in range(C):
        u = np.concatenate([s0[0, c], x[:, c]])
        ref = _silu_math(np.convolve(u, w[c, ::-1], mode="valid"))
        ok &= np.allclose(y[:, c], ref, rtol=0, atol=1e-13)
    out.append(("numpy_convolve", bool(ok)))
    out.append(("state_is_last_rows", np.array_equal(s[0], x[-(d - 1):].T)))
    # one-hot last tap: the convolution is the identity on the current row
    w1 = np.zeros((C, d))
    w1[:, -1] = 1.0
    y1, _ = conv_silu(x, w1, cu, s0)
    out.append(("last_tap_identity", np.allclose(y1, _silu_math(x), rtol=0, atol=1e-14)))
    # one-hot oldest tap: row t sees the input d-1 rows back (the state first)
    w0 = np.zeros((C, d))
    w0[:, 0] = 1.0
    y0, _ = conv_silu(x, w0, cu, s0)
    back = np.concatenate([s0[0].T, x[:T - (d - 1)]])
    out.append(("oldest_tap_delay", np.allclose(y0, _silu_math(back), rtol=0, atol=1e-14)))
    # streaming: rows [0, 4) then [4, T) with the carried state == one pass
    ya, sa = conv_silu(x[:4], w, np.array([0, 4]), s0)
    yb, sb = conv_silu(x[4:], w, np.array([0, T - 4]), sa)
    out.append(("streaming", np.allclose(np.concatenate([ya, yb]), y, rtol=0, atol=1e-14)
                and np.allclose(sb, s, rtol=0, atol=0)))
    # packing: three sequences (one empty, one shorter than the state) == separate runs
    lens = [0, 2, 7]
    cu3 = np.concatenate([[0], np.cumsum(lens)])
    x3 = rng.standard_normal((9, C))
    s3 = rng.standard_normal((3, C, d - 1))
    y3, f3 = conv_silu(x3, w, cu3, s3)
    ok = True
    for i in range(3):
        yi, fi = conv_silu(x3[cu3[i]:cu3[i + 1]], w, np.array([0, lens[i]]), s3[i:i + 1])
        ok &= np.allclose(yi, y3[cu3[i]:cu3[i + 1]], rtol=0, atol=0) and np.array_equal(fi[0], f3[i])
    out.append(("packing", bool(ok)))
    out.append(("empty_passes_state", np.array_equal(f3[0], s3[0])))
    out.append(("short_sequence_state", np.array_equal(f3[1], np.concatenate([s3[1][:, 2:], x3[0:2].T], axis=1))))
    return out


def _conv_reversed_taps(x, w, cu, s0=None):
    return L.conv_silu(x, np.asarray(w)[:, ::-1], cu, s0)


def _conv_reversed_state(x, w, cu, s0=None):
    return L.conv_silu(x, w, cu, None if s0 is None else np.asarray(s0)[:, :, ::-1])


def _conv_ignores_state(x, w, cu, s0=None):
    y, s = L.conv_silu(x, w, cu, None)
    return y, s


def _conv_without_silu(x, w, cu, s0=None):
    y, s = L.conv_silu(x, w, cu, s0)
    # undo SiLU numerically: recompute the plain convolution instead
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    d = w.shape[1]
    N = len(cu) - 1
    s0 = np.zeros((N, x.shape[1], d - 1)) if s0 is None else np.asarray(s0, np.float64)
    for i in range(N):
        u = np.concatenate([s0[i].T, x[cu[i]:cu[i + 1]]])
        for t in range(cu[i + 1] - cu[i]):
            y[cu[i] + t] = sum(w[:, j] * u[t + j] for j in range(d))
    return y, s


def _conv_keeps_first_rows(x, w, cu, s0=None):
    y, s = L.conv_silu(x, w, cu, s0)
    x = np.asarray(x, np.float64)
    N = len(cu) - 1
    d = np.asarray(w).shape[1]
    s0 = np.zeros((N, x.shape[1], d - 1)) if s0 is None else np.asarray(s0, np.float64)
    for i in range(N):
        u = np.concatenate([s0[i].T, x[cu[i]:cu[i + 1]]])
        s[i] = u[:d - 1].T
    return y, s


def test_conv_pins_pass():
    res = conv_pins(L.conv_silu)
    bad = [n for n, ok in res if not ok]
    assert not bad, bad


@pytest.mark.parametrize("mutant", [_conv_reversed_taps, _conv_reversed_state, _conv_ignores_state,
                                    _conv_without_silu, _conv_keeps_first_rows])
def test_conv_mutants_caught(mutant):
    res = conv_pins(mutant)
    assert any(not ok for _, ok in res), mutant.__name__


# ---------------------------------------------------------------------------
# gated RMSNorm
# ---------------------------------------------------------------------------

def norm_pins(gated_rmsnorm):
    out = []
    # hand-worked: o = (3, 4), eps = 0 -> o / sqrt(12.5); z = ln 3 -> silu = ln3 * 3/4
    z = np.full((1, 1, 2), math.log(3.0))
    y = gated_rmsnorm(np.array([[[3.0, 4.0]]]), z, np.array([1.0, 2.0]), 0.0)
    sz = math.log(3.0) * 0.75
    out.append(("hand_values", np.allclose(y[0, 0], [3 / math.sqrt(12.5) * sz, 8 / math.sqrt(12.5) * sz],
                                           rtol=0, atol=1e-14)))
    # epsilon matters for small outputs: o = 1e-4 (3, 4), eps = 1e-6
    y = gated_rmsnorm(np.array([[[3e-4, 4e-4]]]), z, np.array([1.0, 1.0]), 1e-6)
    r = 1.0 / math.sqrt(12.5e-8 + 1e-6)
    out.append(("hand_eps", np.allclose(y[0, 0], [3e-4 * r * sz, 4e-4 * r * sz], rtol=1e-13, atol=0)))
    # torch's rms_norm and silu on random rows (distinct weights per column)
    rng = np.random.default_rng(12)
    o = rng.standard_normal((6, 3, 16))
    zz = rng.standard_normal((6, 3, 16)) * 2
    w = 1 + 0.3 * rng.standard_normal(16)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(o), (16,), torch.from_numpy(w), eps=1e-5) \
        * torch.nn.functional.silu(torch.from_numpy(zz))
    out.append(("torch_rms_norm_silu", np.allclose(gated_rmsnorm(o, zz, w, 1e-5), ref.numpy(),
                                                    rtol=0, atol=1e-13)))
    # rows are independent: changing another head's outputs leaves a row alone
    o2 = o.copy()
    o2[:, 1] *= 5
    a, b = gated_rmsnorm(o, zz, w, 1e-5), gated_rmsnorm(o2, zz, w, 1e-5)
    out.append(("row_independent", np.array_equal(a[:, 0], b[:, 0])))
    return out


def test_norm_pins_pass():
    res = norm_pins(L.gated_rmsnorm)
    bad = [n for n, ok in res if not ok]
    assert not bad, bad


def _norm_sum(o, z, w, eps):
    o = np.asarray(o, np.float64)
    return o / np.sqrt(np.sum(o * o, axis=-1, keepdims=True) + eps) * w * L.silu(z)


def _norm_no_eps(o, z, w, eps):
    return L.gated_rmsnorm(o, z, w, 0.0)


def _norm_silu_on_output(o, z, w, eps):
    o = np.asarray(o, np.float64)
    n = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps) * w
    return L.silu(n) * np.asarray(z, np.float64)


def _norm_no_weight(o, z, w, eps):
    return L.gated_rmsnorm(o, z, np.ones_like(np.asarray(w, np.float64)), eps)


def _norm_over_heads(o, z, w, eps):
    o = np.asarray(o, np.float64)
    ms = np.mean(o * o, axis=(-2, -1), keepdims=True)
    return o / np.sqrt(ms + eps) * w * L.silu(z)


def _norm_sigmoid_gate(o, z, w, eps):
    o = np.asarray(o, np.float64)
    return o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps) * w * oracle.sigmoid(z)


@pytest.mark.parametrize("mutant", [_norm_sum, _norm_no_eps, _norm_silu_on_output, _norm_no_weight,
                                    _norm_over_heads, _norm_sigmoid_gate])
def test_norm_mutants_caught(mutant):
    res = norm_pins(mutant)
    assert any(not ok for _, ok in res), mutant.__name__


# ---------------------------------------------------------------------------
# the whole layer: T = 1 closed form through prologue, operator and epilogue
# ---------------------------------------------------------------------------

def _closed_form_T1(H_k, H_v, d_k, d_v, xr, w, cs, g, beta, S0, z, nw, eps):
    """One token: conv (from the state) + SiLU, then
    o = e^g S0^T q^ + (k^.q^) beta (v - e^g S0^T k^), then the gated norm,
    written out per head with math routines."""
    Cd = xr.shape[0]
    pre = np.array([sum(w[c, j] * (cs[c, j] if j < 3 else xr[c]) for j in range(4)) for c in range(Cd)])
    act = _silu_math(pre)
    nk = H_k * d_k
    out = np.zeros((H_v, d_v))
    for h in range(H_v):
        kh = h // (H_v // H_k)
        q = act[kh * d_k:(kh + 1) * d_k]
        k = act[nk + kh * d_k: nk + (kh + 1) * d_k]
        v = act[2 * nk + h * d_v: 2 * nk + (h + 1) * d_v]
        qh = q / math.sqrt(float(q @ q) + eps) / math.sqrt(d_k)
        kk = k / math.sqrt(float(k @ k) + eps)
        a = math.exp(g[h])
        o = a * (S0[h].T @ qh) + float(kk @ qh) * beta[h] * (v - a * (S0[h].T @ kk))
        rms = math.sqrt(float(o @ o) / d_v + eps)
        out[h] = o / rms * nw * _silu_math(z[h])
    return out


def test_layer_T1_closed_form():
    rng = np.random.default_rng(13)
    H_k, H_v, d_k, d_v = 2, 4, 8, 6
    Cd = 2 * H_k * d_k + H_v * d_v
    xr = rng.standard_normal(Cd)
    w = rng.standard_normal((Cd, 4)) * 0.5
    cs = rng.standard_normal((Cd, 3))
    g = -rng.uniform(0.1, 2.0, H_v)
    beta = rng.uniform(0, 1, H_v)
    S0 = rng.standard_normal((H_v, d_k, d_v)) * 0.3
    z = rng.standard_normal((H_v, d_v))
    nw = 1 + 0.1 * rng.standard_normal(d_v)
    eps = 1e-6
    out, s_fin, c_fin = L.run_layer(H_k, H_v, d_k, d_v, xr[None], w, cs[None], g[None], beta[None],
                                    np.array([0, 1]), S0[None], z[None], nw, eps=eps)
    ref = _closed_form_T1(H_k, H_v, d_k, d_v, xr, w, cs, g, beta, S0, z, nw, eps)
    np.testing.assert_allclose(out[0], ref, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(c_fin[0], np.concatenate([cs[:, 1:], xr[:, None]], axis=1))
    # q and k swapped in the split is a different layer
    q, k, v = L.split_qkv(L.conv_silu(xr[None], w, np.array([0, 1]), cs[None])[0], H_k, H_v, d_k, d_v)
    bad, _ = oracle.run(k, q, v, g[None], beta[None], np.array([0, 1]), S0[None], eps=eps)
    bad = L.gated_rmsnorm(bad, z[None], nw, eps)
    assert np.max(np.abs(bad[0] - ref)) > 1e-3


def test_layer_heads_subset_matches_full():
    rng = np.random.default_rng(14)
    H_k, H_v, d_k, d_v = 1, 2, 8, 8
    Cd = 2 * H_k * d_k + H_v * d_v
    T = 5
    x = rng.standard_normal((T, Cd))
    w = rng.standard_normal((Cd, 4)) * 0.5
    g = -rng.uniform(0.1, 1, (T, H_v))
    b = rng.uniform(0, 1, (T, H_v))
    z = rng.standard_normal((T, H_v, d_v))
    nw = np.ones(d_v)
    full = L.run_layer(H_k, H_v, d_k, d_v, x, w, None, g, b, np.array([0, T]), None, z, nw)
    part = L.run_layer(H_k, H_v, d_k, d_v, x, w, None, g, b, np.array([0, T]), None, z, nw, heads=[1])
    np.testing.assert_array_equal(part[0][:, 1], full[0][:, 1])
    assert not part[0][:, 0].any()
