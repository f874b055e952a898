"""Pins for the fp64 oracle: facts fixed by the mathematics, not by the oracle.

Each ``pin_*`` function runs the oracle (optionally a differently built copy,
``lib``) and returns the largest violation, relative to the size of the
quantity checked.  ``check_all`` runs them all.  The same functions serve the
ordinary pin tests and the mutation tests (which plant single mistakes in
the oracle's C source and require some pin to fail).

Operator (per sequence and value head; "Optimization: Qwen3 next
autoregressive pass (#17996)", build_delta_net_autoregressive):
    q^ = q/|q| * scale, k^ = k/|k|;  S' = e^g S;  delta = beta (v - S'^T k^);
    S = S' + k^ (x) delta;  o = S^T q^.
"""
from __future__ import annotations

import json
import os

import numpy as np

import oracle
from oracle import bruteforce

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

TOL = 1e-9   # fp64 pins: rounding only


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den) if a.size else 0.0


def _rand_inputs(rng, lengths, H_k, H_v, d_k, d_v, decay=(1.0, 16.0),
                 beta=None, s0_std=0.5):
    T = sum(lengths)
    q = rng.standard_normal((T, H_k, d_k)).astype(np.float32)
    k = rng.standard_normal((T, H_k, d_k)).astype(np.float32)
    v = rng.standard_normal((T, H_v, d_v)).astype(np.float32)
    A = rng.uniform(*decay, size=H_v)
    g = (-A[None, :] * np.log1p(np.exp(rng.standard_normal((T, H_v))))).astype(np.float32)
    if beta is None:
        b = (1 / (1 + np.exp(-rng.standard_normal((T, H_v))))).astype(np.float32)
    else:
        b = np.full((T, H_v), beta, np.float32)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    s0 = (rng.standard_normal((len(lengths), H_v, d_k, d_v)) * s0_std) if s0_std else None
    return q, k, v, g, b, cu, s0


def _nrm(x, eps=0.0, factor=1.0):
    x = np.asarray(x, np.float64)
    return x * (factor / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps))


# ---------------------------------------------------------------------------

def pin_t1_closed_form(lib=None):
    """T=1: o = e^g S0^T q^ + (k^.q^) beta (v - e^g S0^T k^); with eps = 0 the new
    state reads beta v + (1-beta) e^g S0^T k^ along k^ and e^g S0^T u along any
    u orthogonal to k^ (the delta rule's defining property)."""
    rng = np.random.default_rng(11)
    H_k, H_v, d = 2, 4, 8
    lengths = [1, 1, 1]
    q, k, v, g, b, cu, s0 = _rand_inputs(rng, lengths, H_k, H_v, d, d)
    out, sf = oracle.recurrent(q, k, v, g, b, cu, s0, eps=0.0, lib_path=lib)
    worst = 0.0
    r = H_v // H_k
    sc = 1 / np.sqrt(d)
    for s in range(3):
        for h in range(H_v):
            qh = _nrm(q[s, h // r], factor=sc)
            kh = _nrm(k[s, h // r])
            a = np.exp(np.float64(g[s, h]))
            bb = np.float64(b[s, h])
            S0 = s0[s, h]
            delta = bb * (v[s, h] - a * S0.T @ kh)
            o = a * S0.T @ qh + (kh @ qh) * delta
            worst = max(worst, _rel(out[s, h], o))
            # along k^: beta v + (1-beta) e^g S0^T k^
            worst = max(worst, _rel(sf[s, h].T @ kh, bb * v[s, h] + (1 - bb) * a * S0.T @ kh))
            # orthogonal complement of k^: untouched apart from the decay
            Qm, _ = np.linalg.qr(np.column_stack([kh, rng.standard_normal((d, d - 1))]))
            U = Qm[:, 1:]
            err = np.max(np.abs(sf[s, h].T @ U - a * S0.T @ U))
            worst = max(worst, float(err / np.max(np.abs(sf[s, h]))))
    # zero initial state: o = beta (k^.q^) v
    out0, _ = oracle.recurrent(q, k, v, g, b, cu, None, eps=0.0, lib_path=lib)
    for s in range(3):
        for h in range(H_v):
            qh = _nrm(q[s, h // r], factor=sc)
            kh = _nrm(k[s, h // r])
            worst = max(worst, _rel(out0[s, h], b[s, h] * (kh @ qh) * v[s, h]))
    return worst


def pin_beta0_pure_decay(lib=None):
    """beta = 0: S_T = e^{sum g} S0 and o_t = e^{G_t} S0^T q^_t."""
    rng = np.random.default_rng(12)
    H_k, H_v, d = 1, 2, 8
    lengths = [9, 4]
    q, k, v, g, b, cu, s0 = _rand_inputs(rng, lengths, H_k, H_v, d, d,
                                         decay=(0.01, 0.2), beta=0.0)
    out, sf = oracle.recurrent(q, k, v, g, b, cu, s0, lib_path=lib)
    worst = 0.0
    for s in range(2):
        a, e = cu[s], cu[s + 1]
        for h in range(H_v):
            G = np.cumsum(g[a:e, h].astype(np.float64))
            worst = max(worst, _rel(sf[s, h], np.exp(G[-1]) * s0[s, h]))
            qh = _nrm(q[a:e, 0], eps=1e-6, factor=1 / np.sqrt(d))
            o = np.exp(G)[:, None] * (qh @ s0[s, h])
            worst = max(worst, _rel(out[a:e, h], o))
    return worst


def _hadamard(n):
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def pin_orthonormal_store(lib=None):
    """g = 0, beta = 1, orthonormal keys, S0 = 0: the state stores each v_s
    under its key (S^T k^_s = v_s), the output is sum_{s<=t} (q^.k^_s) v_s, and
    writing key s again overwrites its value."""
    d = 16
    Hd = _hadamard(d)                       # rows: orthogonal, norm sqrt(d)
    rng = np.random.default_rng(13)
    order = rng.permutation(d)[:10]
    T = 12
    keys = np.concatenate([Hd[order], Hd[order[[3, 7]]]])   # last two repeat
    k = keys.reshape(T, 1, d).astype(np.float32)
    q = rng.standard_normal((T, 1, d)).astype(np.float32)
    v = rng.standard_normal((T, 1, d)).astype(np.float32)
    g = np.zeros((T, 1), np.float32)
    b = np.ones((T, 1), np.float32)
    cu = np.array([0, T], np.int64)
    out, sf = oracle.recurrent(q, k, v, g, b, cu, None, eps=0.0, lib_path=lib)
    kh = keys / np.sqrt(d)
    S = sf[0, 0]
    worst = 0.0
    # latest value stored under each key
    latest = {}
    for t in range(T):
        latest[tuple(keys[t])] = t
    for key, t in latest.items():
        worst = max(worst, _rel(S.T @ (np.array(key) / np.sqrt(d)), v[t, 0]))
    # outputs before any overwrite: sum_{s<=t} (q^.k^_s) v_s
    qh = _nrm(q[:, 0], factor=1 / np.sqrt(d))
    for t in range(10):
        o = sum((qh[t] @ kh[s]) * v[s, 0].astype(np.float64) for s in range(t + 1))
        worst = max(worst, _rel(out[t, 0], o))
    return worst


def pin_golden_hand_example(lib=None):
    """Hand-worked two-token example (tests/golden/hand_example_d2.json)."""
    with open(os.path.join(GOLDEN, "hand_example_d2.json")) as f:
        G = json.load(f)
    q = np.array(G["q"], np.float32).reshape(2, 1, 2)
    k = np.array(G["k"], np.float32).reshape(2, 1, 2)
    v = np.array(G["v"], np.float32).reshape(2, 1, 2)
    g = np.array(G["g"], np.float32).reshape(2, 1)
    b = np.array(G["beta"], np.float32).reshape(2, 1)
    s0 = np.array(G["S0"], np.float64).reshape(1, 1, 2, 2)
    cu = np.array([0, 2], np.int64)
    out, sf = oracle.recurrent(q, k, v, g, b, cu, s0, eps=0.0, lib_path=lib)
    exp_o = np.array(G["expected_out"], np.float64).reshape(2, 1, 2)
    exp_s = np.array(G["expected_state"], np.float64).reshape(1, 1, 2, 2)
    # g = log(1/2) stored in fp32: the decay is 1/2 to ~3e-8 relative
    return max(_rel(out, exp_o), _rel(sf, exp_s)) * (TOL / 1e-6)


def pin_bruteforce(lib=None, chunk=0):
    """Sequential (or chunked) oracle == whole-sequence materialised form."""
    rng = np.random.default_rng(14)
    worst = 0.0
    for lengths, H_k, H_v, d_k, d_v, decay in [
        ([37, 0, 80, 1], 2, 4, 16, 8, (1.0, 16.0)),
        ([150], 1, 2, 8, 16, (0.001, 0.01)),
        ([96, 33], 2, 2, 32, 32, (0.05, 0.5)),
    ]:
        q, k, v, g, b, cu, s0 = _rand_inputs(rng, lengths, H_k, H_v, d_k, d_v, decay=decay)
        if chunk:
            out, sf = oracle.chunked(q, k, v, g, b, cu, s0, chunk=chunk, lib_path=lib)
        else:
            out, sf = oracle.recurrent(q, k, v, g, b, cu, s0, lib_path=lib)
        bo, bs = bruteforce.materialised(q, k, v, g, b, cu, s0)
        worst = max(worst, _rel(out, bo), _rel(sf, bs))
    return worst


def pin_chunked_vs_sequential(lib=None):
    """Chunked WY form == sequential recurrence for C in {1, 7, 16, 64, T}."""
    rng = np.random.default_rng(15)
    lengths = [130, 64, 5]
    q, k, v, g, b, cu, s0 = _rand_inputs(rng, lengths, 2, 4, 16, 16, decay=(0.005, 0.05))
    ref_o, ref_s = oracle.recurrent(q, k, v, g, b, cu, s0, lib_path=lib)
    worst = 0.0
    for C in (1, 7, 16, 64, 130):
        o, s = oracle.chunked(q, k, v, g, b, cu, s0, chunk=C, lib_path=lib)
        worst = max(worst, _rel(o, ref_o), _rel(s, ref_s))
    return worst


SEQUENTIAL_PINS = [pin_t1_closed_form, pin_beta0_pure_decay, pin_orthonormal_store,
                   pin_golden_hand_example, pin_bruteforce]


def check_all(lib=None, chunked_too=True):
    res = {p.__name__: p(lib) for p in SEQUENTIAL_PINS}
    if chunked_too:
        res["pin_chunked_bruteforce"] = pin_bruteforce(lib, chunk=16)
        res["pin_chunked_vs_sequential"] = pin_chunked_vs_sequential(lib)
    return res
