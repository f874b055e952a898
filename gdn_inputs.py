"""Seeded synthetic inputs for the gated DeltaNet operator.

This module is shared by the fp64 oracle's tests, the GPU parity tests and the
benchmark. It draws random numbers and rounds them to the storage dtype; it
holds none of the operator's arithmetic (no decay, no delta rule, no
read-out).

Workload shapes follow the Qwen3-Next linear-attention layer as the pages
describe it ("ik_llama.cpp src/llama-delta-net.cpp", the delta_net
constructor and build_layer_attn_linear_core: key heads H_k, value heads H_v,
head dims d_k = d_v, each key head serving H_v/H_k value heads). The value
distributions are:

* q, k ~ N(0, 1), then scaled to unit L2 norm per head (fp64), then rounded to
  the storage dtype;
* v ~ N(0, 1);
* per value head a decay rate ssm_a = -exp(A_log), A_log = log U(lo, hi)
  (strong decay: lo, hi = 1, 16, the workloads' recipe; weak decay: 0.001,
  0.01), i.e. ssm_a = -U(lo, hi);
* the raw gate projections a, b ~ N(0, 1) per token and value head, and a
  per-head gate bias ssm_dt = 0 (U(-1, 1) with gate_bias=True, to exercise
  the bias input of the in-kernel activations);
* initial states ~ N(0, 0.02) (or zero).

The workloads state the operator's gates as beta = sigmoid(b) and
g = ssm_a * softplus(a + ssm_dt) of these draws.  Those two functions are
the layer's gate activations, part of the method under test when the kernels
apply them (gate_mode GDN_GATES_RAW), so this module does not evaluate them:
a caller that wants the final gates passes `final_gates(a, b, ssm_a, ssm_dt)
-> (g, beta)`, evaluated by the test or benchmark harness.  Without it, g and
beta are None and only the raw projections are available.  beta_mode
"zero"/"one" and decay "zero" (g = 0) set the final gates directly.

Draw order is fixed: ssm_a, q, k, v, a, b, [ssm_dt], initial states, slots.
bf16 storage is round-to-nearest-even of the fp32 value; arrays are returned as float32 numpy arrays that hold the exactly rounded values, so the
oracle (which upcasts to fp64) and the GPU (which converts to bf16 without
further rounding) consume identical numbers.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

QWEN3_NEXT_HEADS = dict(H_k=16, H_v=32, d_k=128, d_v=128)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    r = ((u + bias) & np.uint64(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    # input recipe: unit L2 norm per head vector, in fp64
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / n


@dataclasses.dataclass
class Case:
    """One prefill workload: packed varlen tokens + a pool of state slots."""
    name: str
    H_k: int
    H_v: int
    d_k: int
    d_v: int
    dtype: str                 # "f32" or "bf16": storage dtype of q, k, v, out
    lengths: List[int]
    q: np.ndarray              # [T][H_k][d_k] float32 (values exact in dtype)
    k: np.ndarray              # [T][H_k][d_k]
    v: np.ndarray              # [T][H_v][d_v]
    g: Optional[np.ndarray]    # [T][H_v] float32, log-decay <= 0 (None: not evaluated)
    beta: Optional[np.ndarray]  # [T][H_v] float32 in [0, 1] (None: not evaluated)
    pool: np.ndarray           # [n_slots][H_v][d_k][d_v] float32 initial state pool
    slot_in: np.ndarray        # [N] int32 (-1 = zero initial state)
    slot_out: np.ndarray       # [N] int32
    ssm_a: np.ndarray          # [H_v] float32 decay rate (<= 0)
    raw_a: np.ndarray          # [T][H_v] float32 raw gate projection
    raw_b: np.ndarray          # [T][H_v] float32 raw write-strength projection
    ssm_dt: np.ndarray         # [H_v] float32 gate bias (zero unless gate_bias)

    @property
    def n_seqs(self) -> int:
        return len(self.lengths)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.lengths))

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int32)


def _draw(rng, T, H_k, H_v, d_k, d_v, dtype, decay, beta_mode, a_lo, a_hi,
          final_gates=None, gate_bias=False):
    if decay == "strong":
        ssm_a = -rng.uniform(1.0, 16.0, size=H_v)
    elif decay == "weak":
        ssm_a = -rng.uniform(0.001, 0.01, size=H_v)
    elif decay == "custom":
        ssm_a = -rng.uniform(a_lo, a_hi, size=H_v)
    elif decay == "zero":
        ssm_a = np.zeros(H_v)
    else:
        raise ValueError(decay)
    if beta_mode not in ("random", "zero", "one"):
        raise ValueError(beta_mode)
    q = _unit_rows(rng.standard_normal((T, H_k, d_k)))
    k = _unit_rows(rng.standard_normal((T, H_k, d_k)))
    v = rng.standard_normal((T, H_v, d_v))
    raw_a = rng.standard_normal((T, H_v))
    raw_b = rng.standard_normal((T, H_v))
    ssm_dt = rng.uniform(-1.0, 1.0, size=H_v) if gate_bias else np.zeros(H_v)
    f32 = lambda x: np.ascontiguousarray(x, dtype=np.float32)
    ssm_a, raw_a, raw_b, ssm_dt = f32(ssm_a), f32(raw_a), f32(raw_b), f32(ssm_dt)
    g = beta = None
    if final_gates is not None:
        g, beta = final_gates(raw_a, raw_b, ssm_a, ssm_dt)
        g, beta = f32(g), f32(beta)
    if decay == "zero":
        g = np.zeros((T, H_v), np.float32)
    if beta_mode == "zero":
        beta = np.zeros((T, H_v), np.float32)
    elif beta_mode == "one":
        beta = np.ones((T, H_v), np.float32)
    q = q.astype(np.float32)
    k = k.astype(np.float32)
    v = v.astype(np.float32)
    if dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    elif dtype != "f32":
        raise ValueError(dtype)
    return (ssm_a, q, k, v, g, beta, raw_a, raw_b, ssm_dt)


def make_case(name: str, lengths, H_k: int, H_v: int, d_k: int, d_v: int,
              dtype: str, seed: int, decay: str = "strong",
              beta_mode: str = "random", s0_std: float = 0.02,
              n_slots: Optional[int] = None, scatter_slots: bool = False,
              a_lo: float = 1.0, a_hi: float = 16.0, final_gates=None,
              gate_bias: bool = False) -> Case:
    """Generic generator. s0_std == 0 gives zero initial states (slot_in = -1).
    final_gates: see the module docstring (None leaves g and beta unset)."""
    lengths = [int(x) for x in lengths]
    N = len(lengths)
    T = int(sum(lengths))
    rng = np.random.default_rng(seed)
    ssm_a, q, k, v, g, beta, raw_a, raw_b, ssm_dt = _draw(
        rng, T, H_k, H_v, d_k, d_v, dtype, decay, beta_mode, a_lo, a_hi, final_gates, gate_bias)
    if n_slots is None:
        n_slots = N
    if s0_std > 0:
        pool = (rng.standard_normal((n_slots, H_v, d_k, d_v)) * s0_std).astype(np.float32)
    else:
        pool = np.zeros((n_slots, H_v, d_k, d_v), np.float32)
    if scatter_slots:
        perm = rng.permutation(n_slots)[:N]
        slots = perm.astype(np.int32)
    else:
        slots = np.arange(N, dtype=np.int32)
    slot_in = slots.copy() if s0_std > 0 else np.full(N, -1, np.int32)
    return Case(name, H_k, H_v, d_k, d_v, dtype, lengths, q, k, v, g, beta,
                pool, slot_in, slots.copy(), ssm_a, raw_a, raw_b, ssm_dt)


# ---------------------------------------------------------------------------
# The five named workloads (seed = workload index) and the stress sets.
# ---------------------------------------------------------------------------

def config0(final_gates=None) -> Case:
    """Tiny fp32 case: 1 sequence, T=128, H_k=H_v=2, d=32, zero initial state."""
    return make_case("tiny_f32_T128", [128], 2, 2, 32, 32, "f32", seed=0, s0_std=0.0,
                     final_gates=final_gates)


def config1(T: int = 4096, final_gates=None) -> Case:
    """Single-layer prefill: 1 sequence, T=4096, Qwen3-Next heads, bf16."""
    return make_case(f"prefill_T{T}", [T], dtype="bf16", seed=1, final_gates=final_gates,
                     **QWEN3_NEXT_HEADS)


CONFIG3_LENGTHS = [17, 64, 65, 300, 512, 1023, 2048, 8192]


def config3(final_gates=None) -> Case:
    """Mixed varlen batch: 8 sequences, scattered slots in a 64-slot pool."""
    return make_case("varlen8_T12221", CONFIG3_LENGTHS, dtype="bf16", seed=3,
                     n_slots=64, scatter_slots=True, final_gates=final_gates,
                     **QWEN3_NEXT_HEADS)


def config4(T: int = 65536, final_gates=None) -> Case:
    """Long context: 1 sequence of 65536 tokens (fed as 128 ubatches of 512)."""
    return make_case(f"stream_T{T}", [T], dtype="bf16", seed=4, final_gates=final_gates,
                     **QWEN3_NEXT_HEADS)


@dataclasses.dataclass
class DecodeCase:
    """Autoregressive workload: n_steps steps of one token for each of n_seqs."""
    name: str
    H_k: int
    H_v: int
    d_k: int
    d_v: int
    dtype: str
    n_seqs: int
    n_steps: int
    q: np.ndarray      # [steps][N][H_k][d_k]
    k: np.ndarray      # [steps][N][H_k][d_k]
    v: np.ndarray      # [steps][N][H_v][d_v]
    g: np.ndarray      # [steps][N][H_v]
    beta: np.ndarray   # [steps][N][H_v]
    pool: np.ndarray   # [n_slots][H_v][d_k][d_v]
    slots: np.ndarray  # [N] int32: slot of sequence i (read and written in place)
    ssm_a: np.ndarray  # [H_v] decay rate (<= 0)
    raw_a: np.ndarray  # [steps][N][H_v] raw gate projection
    raw_b: np.ndarray  # [steps][N][H_v] raw write-strength projection
    ssm_dt: np.ndarray  # [H_v] gate bias


def make_decode(name: str, n_seqs: int, n_steps: int, H_k: int, H_v: int,
                d_k: int, d_v: int, dtype: str, seed: int,
                decay: str = "strong", beta_mode: str = "random",
                s0_std: float = 0.02, n_slots: Optional[int] = None,
                scatter_slots: bool = False, final_gates=None,
                gate_bias: bool = False) -> DecodeCase:
    rng = np.random.default_rng(seed)
    ssm_a, q, k, v, g, beta, raw_a, raw_b, ssm_dt = _draw(
        rng, n_steps * n_seqs, H_k, H_v, d_k, d_v, dtype, decay, beta_mode, 1.0, 16.0,
        final_gates, gate_bias)
    if n_slots is None:
        n_slots = n_seqs
    pool = (rng.standard_normal((n_slots, H_v, d_k, d_v)) * s0_std).astype(np.float32)
    if scatter_slots:
        slots = rng.permutation(n_slots)[:n_seqs].astype(np.int32)
    else:
        slots = np.arange(n_seqs, dtype=np.int32)
    S, N = n_steps, n_seqs
    return DecodeCase(name, H_k, H_v, d_k, d_v, dtype, N, S,
                      q.reshape(S, N, H_k, d_k), k.reshape(S, N, H_k, d_k),
                      v.reshape(S, N, H_v, d_v),
                      None if g is None else g.reshape(S, N, H_v),
                      None if beta is None else beta.reshape(S, N, H_v), pool, slots, ssm_a,
                      raw_a.reshape(S, N, H_v), raw_b.reshape(S, N, H_v), ssm_dt)


def config2(n_steps: int = 128, final_gates=None) -> DecodeCase:
    """Decode: 64 sequences x 128 steps, Qwen3-Next heads, bf16, 128 MiB pool."""
    return make_decode("decode64x128", 64, n_steps, dtype="bf16", seed=2,
                       final_gates=final_gates, **QWEN3_NEXT_HEADS)


def decode_as_sequences(dc: DecodeCase):
    """Re-pack a decode workload as N sequences of n_steps tokens (seq-major).

    Returns (q, k, v, g, beta, cu_seqlens) in the packed varlen layout, with
    sequence i holding steps 0..n_steps-1 of decode sequence i.
    """
    perm = lambda a: np.ascontiguousarray(np.swapaxes(a, 0, 1)).reshape((-1,) + a.shape[2:])
    cu = (np.arange(dc.n_seqs + 1) * dc.n_steps).astype(np.int32)
    return perm(dc.q), perm(dc.k), perm(dc.v), perm(dc.g), perm(dc.beta), cu


# ---------------------------------------------------------------------------
# Layer inputs for the fused prologue / epilogue ("ik_llama.cpp
# src/llama-delta-net.cpp", build_layer_attn_linear_core): the mixed q|k|v
# projection rows that the short causal convolution reads, its taps and
# per-slot convolution states, and the gate z and weight of the gated RMSNorm.
# ---------------------------------------------------------------------------

D_CONV = 4      # taps of the short convolution


@dataclasses.dataclass
class LayerInputs:
    qkv: np.ndarray        # [T][conv_dim] float32 (exact in dtype): q channels, k channels, v channels
    conv_w: np.ndarray     # [conv_dim][D_CONV] float32, oldest tap first
    conv_pool: np.ndarray  # [n_slots][conv_dim][D_CONV-1] float32 (exact in dtype), oldest first
    z: np.ndarray          # [T][H_v][d_v] float32 (exact in dtype)
    norm_w: np.ndarray     # [d_v] float32


def conv_dim(H_k: int, H_v: int, d_k: int, d_v: int) -> int:
    return 2 * H_k * d_k + H_v * d_v


def make_layer_inputs(T: int, n_slots: int, H_k: int, H_v: int, d_k: int, d_v: int,
                      dtype: str, seed: int, w_std: float = 0.5) -> LayerInputs:
    """Draws, from a stream of their own (so a workload's other inputs are
    unchanged): qkv rows ~ N(0, 1); taps ~ N(0, w_std^2) (w_std = 0.5 keeps the
    convolution's output near unit variance); convolution states ~ N(0, 1)
    (they hold earlier rows); z ~ N(0, 1); norm weight 1 + 0.1 N(0, 1)."""
    rng = np.random.default_rng([seed, 7])
    C = conv_dim(H_k, H_v, d_k, d_v)
    qkv = rng.standard_normal((T, C)).astype(np.float32)
    conv_w = (rng.standard_normal((C, D_CONV)) * w_std).astype(np.float32)
    conv_pool = rng.standard_normal((n_slots, C, D_CONV - 1)).astype(np.float32)
    z = rng.standard_normal((T, H_v, d_v)).astype(np.float32)
    norm_w = (1.0 + 0.1 * rng.standard_normal(d_v)).astype(np.float32)
    if dtype == "bf16":
        qkv, conv_pool, z = round_to_bf16(qkv), round_to_bf16(conv_pool), round_to_bf16(z)
    return LayerInputs(qkv, conv_w, conv_pool, z, norm_w)
