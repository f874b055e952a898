"""fp64 CPU oracle for the gated DeltaNet operator -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its Python binding) never
does, and shares no code with it.

* ``recurrent(...)``: the plain definition, token by token in fp64 (C,
  ``gdn_oracle.c``), threaded over independent (sequence, value head) chains.
* ``chunked(...)``: the same operator in the chunked WY form of the pages'
  chunked graph, in fp64 (C), for the chunked-vs-sequential pin.
* ``chunk_dump(...)``: the chunked form for one value head, returning the
  intermediates (g_cumsum, T, k_cumdecay, v_new) of the chunk holding a given
  token, for comparison with the library's debug record.
* ``bruteforce.materialised(...)``: the whole-sequence O(T^2) materialised
  form solved with a library triangular solver (numpy/scipy).
* ``gates(...)``: the gate activations of the layer (raw projections to the
  operator's g and beta), in fp64.
* ``layer``: the steps of the layer right before and after the operator (the
  short causal convolution + SiLU prologue with its per-slot state, the gated
  RMSNorm epilogue) and ``layer.run_layer`` chaining them around ``run``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the C oracle with gcc (plain -O2, no fast-math)."""
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c99", "-pthread",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: Optional[str] = None) -> ctypes.CDLL:
    path = path or _LIB
    if not os.path.exists(path):
        build(out=path)
    lib = ctypes.CDLL(path)
    f = lib.gdn_oracle_run
    P = ctypes.c_void_p
    f.argtypes = [ctypes.c_int32, P, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, P,
                  ctypes.c_double, ctypes.c_double, P, ctypes.c_int32, P, P,
                  ctypes.c_int32, ctypes.c_int32]
    f.restype = ctypes.c_int
    d = lib.gdn_oracle_chunk_dump
    d.argtypes = [ctypes.c_int32, P, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, P,
                  ctypes.c_double, ctypes.c_double, ctypes.c_int32, ctypes.c_int64,
                  ctypes.c_int32, P, P, P, P, P, P, P]
    d.restype = ctypes.c_int
    return lib


_lib_cache = {}


def _get(path: Optional[str]) -> ctypes.CDLL:
    key = path or _LIB
    if key not in _lib_cache:
        _lib_cache[key] = load(path)
    return _lib_cache[key]


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def softplus(x):
    """log(1 + e^x) in fp64, written as max(x, 0) + log1p(e^-|x|) so that
    neither branch overflows."""
    x = np.asarray(x, np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    """1 / (1 + e^-x) in fp64, evaluated through e^-|x| (no overflow)."""
    x = np.asarray(x, np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def gates(a, b, ssm_a, ssm_dt):
    """The layer's gate activations ("Optimization: Qwen3 next autoregressive
    pass (#17996)", build_layer_attn_linear): beta = sigmoid(b) and
    gate = softplus(a + ssm_dt) * ssm_a, with the per-value-head bias ssm_dt
    and decay rate ssm_a (<= 0) broadcast over tokens.  a, b: [T, H_v];
    returns (g, beta) [T, H_v] in fp64."""
    a = np.asarray(a, np.float64)
    g = softplus(a + np.asarray(ssm_dt, np.float64)[None, :]) * np.asarray(ssm_a, np.float64)[None, :]
    return g, sigmoid(b)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def run(q, k, v, g, beta, cu_seqlens, s0=None, *, scale: Optional[float] = None,
        eps: float = 1e-6, heads: Optional[Sequence[int]] = None, chunk: int = 0,
        threads: Optional[int] = None, lib_path: Optional[str] = None):
    """Run the oracle over a packed varlen batch.

    q, k: [T, H_k, d_k]; v: [T, H_v, d_v]; g, beta: [T, H_v]; cu_seqlens:
    [N+1]; s0: [N, H_v, d_k, d_v] initial states (None = zero).  Returns
    (out [T, H_v, d_v] fp64, s_final [N, H_v, d_k, d_v] fp64).  With
    ``heads``, only those value heads are computed (others are zero).
    chunk=0 is the sequential recurrence; chunk>0 the chunked WY form.
    """
    q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
    T, H_k, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    assert k.shape == q.shape and v.shape[0] == T
    assert g.shape == (T, H_v) and beta.shape == (T, H_v)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    assert cu[-1] == T
    if scale is None:
        scale = 1.0 / np.sqrt(d_k)
    if s0 is not None:
        s0 = np.ascontiguousarray(s0, dtype=np.float64)
        assert s0.shape == (N, H_v, d_k, d_v)
    if heads is not None:
        hl = np.ascontiguousarray(heads, dtype=np.int32)
        nh = hl.shape[0]
    else:
        hl, nh = None, 0
    out = np.zeros((T, H_v, d_v), np.float64)
    s_out = np.zeros((N, H_v, d_k, d_v), np.float64)
    nthreads = threads or default_threads()
    rc = _get(lib_path).gdn_oracle_run(
        N, _ptr(cu), H_k, H_v, d_k, d_v, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
        _ptr(beta), _ptr(s0), float(scale), float(eps), _ptr(hl), nh,
        _ptr(out), _ptr(s_out), int(chunk), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    return out, s_out


def chunk_dump(q, k, v, g, beta, cu_seqlens, s0=None, *, token: int, head: int,
               scale: Optional[float] = None, eps: float = 1e-6, chunk: int = 64,
               lib_path: Optional[str] = None) -> dict:
    """The chunked form for value head ``head`` with the intermediates of the
    chunk holding packed token ``token``: a dict with t0 and len (0 when no
    chunk holds it), G [len], T [len, len], W [len, d_k] (k_cumdecay) and
    U [len, d_v] (v_new), all fp64, plus that head's out and final states."""
    q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
    T, H_k, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    assert cu[-1] == T
    if scale is None:
        scale = 1.0 / np.sqrt(d_k)
    if s0 is not None:
        s0 = np.ascontiguousarray(s0, dtype=np.float64)
        assert s0.shape == (N, H_v, d_k, d_v)
    out = np.zeros((T, H_v, d_v), np.float64)
    s_out = np.zeros((N, H_v, d_k, d_v), np.float64)
    G = np.zeros(chunk, np.float64)
    Tm = np.zeros((chunk, chunk), np.float64)
    W = np.zeros((chunk, d_k), np.float64)
    U = np.zeros((chunk, d_v), np.float64)
    meta = np.zeros(2, np.int64)
    rc = _get(lib_path).gdn_oracle_chunk_dump(
        N, _ptr(cu), H_k, H_v, d_k, d_v, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
        _ptr(beta), _ptr(s0), float(scale), float(eps), int(chunk), int(token), int(head),
        _ptr(out), _ptr(s_out), _ptr(G), _ptr(Tm), _ptr(W), _ptr(U), _ptr(meta))
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    n = int(meta[1])
    return {"t0": int(meta[0]), "len": n, "G": G[:n].copy(), "T": Tm[:n, :n].copy(),
            "W": W[:n].copy(), "U": U[:n].copy(), "out": out[:, head], "s_out": s_out[:, head]}


def recurrent(*args, **kw):
    """Sequential fp64 recurrence (the plain definition)."""
    kw["chunk"] = 0
    return run(*args, **kw)


def chunked(*args, chunk: int = 64, **kw):
    """Chunked WY form in fp64 (the pages' chunked graph)."""
    assert chunk > 0
    kw["chunk"] = chunk
    return run(*args, **kw)


def run_case(case, heads=None, threads=None, chunk: int = 0, lib_path=None,
             raw_gates: bool = False):
    """Oracle on a gdn_inputs.Case: maps slots to per-sequence initial states.
    With raw_gates, g and beta come from the case's raw projections through
    ``gates`` (the in-kernel activation path) instead of the case's g, beta."""
    N = case.n_seqs
    s0 = np.zeros((N, case.H_v, case.d_k, case.d_v), np.float64)
    for i in range(N):
        if case.slot_in[i] >= 0:
            s0[i] = case.pool[case.slot_in[i]]
    g, beta = case.g, case.beta
    if raw_gates:
        g, beta = gates(case.raw_a, case.raw_b, case.ssm_a, case.ssm_dt)
    return run(case.q, case.k, case.v, g, beta, case.cu_seqlens, s0,
               heads=heads, threads=threads, chunk=chunk, lib_path=lib_path)
