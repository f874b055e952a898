"""fp64 oracle of the layer steps around the operator -- TEST INFRASTRUCTURE
(only the tests, the smoke check and the benchmark's CPU-baseline leg use it).

What the Qwen3-Next linear-attention layer does right before and right after
the gated delta rule, as build_layer_attn_linear_core on the page
"ik_llama.cpp src/llama-delta-net.cpp" builds it:

* prologue (``conv_silu``): ggml_ssm_conv over the mixed q|k|v projection rows
  with the per-slot convolution state, then ggml_silu; the result is viewed as
  q (first H_k*d_k channels), k (next H_k*d_k) and v (last H_v*d_v); the new
  convolution state is the last d_conv - 1 inputs.
* epilogue (``gated_rmsnorm``): llm_build_norm with LLM_NORM_RMS and the
  ssm_norm weight over each (token, value head) row of d_v outputs, then
  ggml_fused_mul_unary(z, ., SILU), i.e. times silu(z).

Readings where the page leaves a step open:
* the convolution taps are stored [channel][d_conv] with the oldest tap first,
  so the last tap multiplies the current row (a causal depthwise
  convolution; the state layout [channel][d_conv - 1] of the page's
  conv_states view, oldest first, is the same time order);
* RMS norm: x / sqrt(mean(x^2) + eps) * weight with the layer's norm epsilon
  (the same f_norm_rms_eps the page passes to the L2 norms).

Everything here is plain fp64 numpy, token by token where the layer is
sequential.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from . import run, sigmoid


def silu(x):
    """x * sigmoid(x) in fp64."""
    x = np.asarray(x, np.float64)
    return x * sigmoid(x)


def conv_silu(x, w, cu_seqlens, s0=None):
    """Causal depthwise convolution + SiLU over packed varlen rows.

    x: [T, C] input rows; w: [C, d] taps, oldest first; cu_seqlens: [N+1];
    s0: [N, C, d-1] convolution state of each sequence (the d-1 inputs before
    its first row, oldest first; None = zeros).  For sequence i with rows
    u = s0[i]^T followed by its own rows, output row t is
    silu(sum_j w[:, j] * u[t + j]).  Returns (y [T, C], s_final [N, C, d-1])
    in fp64, s_final holding the last d-1 rows of u.
    """
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    cu = np.asarray(cu_seqlens, np.int64)
    T, C = x.shape
    d = w.shape[1]
    N = cu.shape[0] - 1
    if s0 is None:
        s0 = np.zeros((N, C, d - 1))
    s0 = np.asarray(s0, np.float64)
    y = np.zeros((T, C))
    s_fin = np.zeros((N, C, d - 1))
    for i in range(N):
        tb, te = int(cu[i]), int(cu[i + 1])
        u = np.concatenate([s0[i].T, x[tb:te]], axis=0)       # [d-1+len, C], time order
        for t in range(te - tb):
            acc = np.zeros(C)
            for j in range(d):
                acc += w[:, j] * u[t + j]
            y[tb + t] = silu(acc)
        s_fin[i] = u[te - tb: te - tb + d - 1].T
    return y, s_fin


def split_qkv(y, H_k, H_v, d_k, d_v):
    """The q, k, v views of the convolution output (channel order q | k | v)."""
    T = y.shape[0]
    nk = H_k * d_k
    q = y[:, :nk].reshape(T, H_k, d_k)
    k = y[:, nk:2 * nk].reshape(T, H_k, d_k)
    v = y[:, 2 * nk:].reshape(T, H_v, d_v)
    return q, k, v


def gated_rmsnorm(o, z, w, eps):
    """rms_norm(o) * w * silu(z) over the last axis (d_v), in fp64."""
    o = np.asarray(o, np.float64)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    return o / np.sqrt(ms + eps) * np.asarray(w, np.float64) * silu(z)


def run_layer(H_k, H_v, d_k, d_v, qkv, conv_w, conv_s0, g, beta, cu_seqlens, s0=None,
              z=None, norm_w=None, *, scale: Optional[float] = None, eps: float = 1e-6,
              heads: Optional[Sequence[int]] = None, threads: Optional[int] = None):
    """Prologue -> gated delta rule (``oracle.run``) -> optional epilogue.

    Returns (out [T, H_v, d_v], s_final [N, H_v, d_k, d_v],
    conv_final [N, conv_dim, d_conv-1]), all fp64.  With ``heads`` only those
    value heads are computed (the others' outputs are zero).
    """
    y, conv_fin = conv_silu(qkv, conv_w, cu_seqlens, conv_s0)
    q, k, v = split_qkv(y, H_k, H_v, d_k, d_v)
    out, s_fin = run(q, k, v, g, beta, cu_seqlens, s0, scale=scale, eps=eps, heads=heads,
                     threads=threads)
    if z is not None:
        out = gated_rmsnorm(out, z, norm_w, eps)
        if heads is not None:
            mask = np.zeros(H_v, bool)
            mask[list(heads)] = True
            out[:, ~mask] = 0.0
    return out, s_fin, conv_fin
