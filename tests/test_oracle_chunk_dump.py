"""Pins of the oracle's chunk record (oracle.chunk_dump), the reference the
library's GDN_DEBUG_DUMP record is compared with.  Each intermediate of the
chunked form (build_delta_net_chunking on "Optimization: Qwen3 next
autoregressive pass (#17996)": g_cumsum, the solved attn, k_cumdecay, v_new)
is checked against its definition computed another way: T against a library
matrix inverse of I + A, and v_new against the state the sequential
recurrence reaches at the chunk's first token."""
import numpy as np
import pytest

import oracle
import workloads as gi


def _norm(x, eps=1e-6):
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + eps)


@pytest.mark.parametrize("seq,offset", [(0, 5), (1, 70), (2, 0)])
def test_chunk_record_matches_definitions(seq, offset):
    case = gi.make_case("dump_pin", [100, 150, 64], 1, 2, 16, 8, "f32", seed=31)
    cu = case.cu_seqlens.astype(np.int64)
    token, head = int(cu[seq] + offset), 1
    s0 = np.stack([case.pool[s] if s >= 0 else np.zeros_like(case.pool[0]) for s in case.slot_in])
    rec = oracle.chunk_dump(case.q, case.k, case.v, case.g, case.beta, cu, s0, token=token, head=head)
    t0 = int(cu[seq] + (offset // 64) * 64)
    n = int(min(64, cu[seq + 1] - t0))
    assert rec["t0"] == t0 and rec["len"] == n
    r = case.H_v // case.H_k
    q = _norm(case.q[t0:t0 + n, head // r].astype(np.float64)) / np.sqrt(case.d_k)
    k = _norm(case.k[t0:t0 + n, head // r].astype(np.float64))
    v = case.v[t0:t0 + n, head].astype(np.float64)
    g = case.g[t0:t0 + n, head].astype(np.float64)
    b = case.beta[t0:t0 + n, head].astype(np.float64)
    G = np.cumsum(g)
    np.testing.assert_allclose(rec["G"], G, rtol=0, atol=1e-12 * (1 + np.abs(G).max()))
    decay = np.tril(np.exp(G[:, None] - G[None, :]))
    A = np.tril(b[:, None] * (k @ k.T) * decay, -1)
    T = np.linalg.inv(np.eye(n) + A)
    np.testing.assert_allclose(rec["T"], T, rtol=0, atol=1e-10 * np.abs(T).max())
    W = T @ ((b * np.exp(G))[:, None] * k)
    np.testing.assert_allclose(rec["W"], W, rtol=0, atol=1e-10 * np.abs(W).max())
    # the state entering the chunk, from the sequential recurrence over the
    # sequence's tokens before t0
    s_in = s0[seq, head].astype(np.float64)
    if t0 > cu[seq]:
        a, e = int(cu[seq]), t0
        _, st = oracle.recurrent(case.q[a:e], case.k[a:e], case.v[a:e], case.g[a:e], case.beta[a:e],
                                 np.array([0, e - a]), s0[seq:seq + 1])
        s_in = st[0, head]
    U = T @ (b[:, None] * v) - W @ s_in
    np.testing.assert_allclose(rec["U"], U, rtol=0, atol=1e-10 * np.abs(U).max())
    # the read-out of the chunk from the record: (e^G q^) S + (q^ k^T * decay) U
    out = (np.exp(G)[:, None] * q) @ s_in + (np.tril(q @ k.T) * decay) @ rec["U"]
    np.testing.assert_allclose(rec["out"][t0:t0 + n], out, rtol=0, atol=1e-10 * np.abs(out).max())


def test_chunk_record_of_a_token_outside_the_batch_is_empty():
    case = gi.make_case("dump_none", [40], 1, 1, 16, 16, "f32", seed=32)
    rec = oracle.chunk_dump(case.q, case.k, case.v, case.g, case.beta, case.cu_seqlens, token=40, head=0)
    assert rec["len"] == 0 and rec["G"].size == 0
