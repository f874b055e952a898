"""Python binding of libgdn (the gated DeltaNet operator on MI355X).

Argument marshalling only: every step of the operator runs in the HIP kernels
of ``libgdn.so``.  PyTorch supplies device memory and the current stream.
There is no fallback: if the library is missing this module raises on import.

    import gated_deltanet_rule_amd as gdn
    gdn.prefill(q, k, v, g, beta, state_in, state_out, out, cu_seqlens, slot_in, slot_out)
    gdn.decode_step(q, k, v, g, beta, state_in, state_out, out, slot_in, slot_out)

Shapes: q, k [T, H_k, d_k]; v, out [T, H_v, d_v]; g, beta [T, H_v] fp32;
state pools fp32 [n_slots, H_v, d_k, d_v]; cu_seqlens [N+1], slot_in/slot_out
[N] int32 on the device.  q/k/v are all fp32 or all bf16; out is fp32 or
bf16 independently (its dtype selects the output type).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_OK = 0
GDN_F32 = 0
GDN_BF16 = 1
GDN_GATES_FINAL = 0
GDN_GATES_RAW = 1
D_CONV = 4          # taps of the fused convolution prologue


class GdnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libgdn status {status}: {msg}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("H_k", ctypes.c_int32), ("H_v", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("slot_stride", ctypes.c_int64), ("scale", ctypes.c_float),
                ("eps", ctypes.c_float), ("gate_mode", ctypes.c_int32),
                ("ssm_a", ctypes.c_void_p), ("ssm_dt", ctypes.c_void_p),
                ("d_conv", ctypes.c_int32), ("conv_w", ctypes.c_void_p),
                ("z", ctypes.c_void_p), ("norm_w", ctypes.c_void_p),
                ("n_slots", ctypes.c_int32)]


class DebugChunk(ctypes.Structure):
    """gdn_debug_chunk: one chunk's intermediates recorded under GDN_DEBUG_DUMP."""
    _fields_ = [("token", ctypes.c_int32), ("head", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("t0", ctypes.c_int32), ("len", ctypes.c_int32), ("d_k", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("prepared", ctypes.c_int32), ("scanned", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("G", ctypes.c_double * 64),
                ("T", ctypes.c_float * (64 * 64)), ("W", ctypes.c_float * (64 * 128)),
                ("U", ctypes.c_float * (64 * 128))]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libgdn.so not built at {LIB_PATH}; run "
                          "`python gated_deltanet_rule_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D = ctypes.POINTER(Dims)
    lib.gdn_version.restype = ctypes.c_int
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_prefill_workspace_size.argtypes = [D, I32, I64, ctypes.POINTER(SZ)]
    lib.gdn_prefill_workspace_size.restype = ctypes.c_int
    lib.gdn_chunked_prefill_workspace_size.argtypes = [D, I32, I64, ctypes.POINTER(SZ)]
    lib.gdn_chunked_prefill_workspace_size.restype = ctypes.c_int
    lib.gdn_chunked_prefill.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, I32, I64, P, SZ, P]
    lib.gdn_chunked_prefill.restype = ctypes.c_int
    lib.gdn_chunked_prefill_noalloc.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, I32, I64, P]
    lib.gdn_chunked_prefill_noalloc.restype = ctypes.c_int
    lib.gdn_recurrent_step.argtypes = [D, P, P, P, P, P, P, P, P, P, P, I32, P]
    lib.gdn_recurrent_step.restype = ctypes.c_int
    lib.gdn_prefill_prepare.argtypes = [D, P, P, P, P, P, P, I32, I64, P, SZ, P]
    lib.gdn_prefill_prepare.restype = ctypes.c_int
    lib.gdn_prefill_scan.argtypes = [D, P, P, P, P, P, I32, I64, P, SZ, P]
    lib.gdn_prefill_scan.restype = ctypes.c_int
    lib.gdn_recurrent_multi.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, I32, I64, P]
    lib.gdn_recurrent_multi.restype = ctypes.c_int
    lib.gdn_debug_dump.argtypes = [ctypes.POINTER(DebugChunk)]
    lib.gdn_debug_dump.restype = ctypes.c_int
    return lib


lib = _load()

EXPORTED = ["gdn_version", "gdn_status_string", "gdn_last_error",
            "gdn_prefill_workspace_size", "gdn_chunked_prefill_workspace_size",
            "gdn_chunked_prefill", "gdn_chunked_prefill_noalloc", "gdn_prefill_prepare",
            "gdn_prefill_scan", "gdn_recurrent_step", "gdn_recurrent_multi", "gdn_debug_dump"]


def version() -> int:
    return lib.gdn_version()


def debug_dump() -> dict:
    """The last chunk recorded under GDN_DEBUG_DUMP=<token>,<head>: the
    header fields, and as float64 arrays the valid parts G[len], T[len][len],
    W[len][d_k] and U[len][d_v] (absent when not written).  Raises GdnError
    when no prefill has run with the variable set."""
    import numpy as np
    rec = DebugChunk()
    _check(lib.gdn_debug_dump(ctypes.byref(rec)))
    out = {f: getattr(rec, f) for f in ("token", "head", "chunk", "t0", "len", "d_k", "d_v",
                                        "prepared", "scanned")}
    n = rec.len
    if rec.prepared:
        out["G"] = np.ctypeslib.as_array(rec.G)[:n].astype(np.float64)
        out["T"] = np.ctypeslib.as_array(rec.T).reshape(64, 64)[:n, :n].astype(np.float64)
        out["W"] = np.ctypeslib.as_array(rec.W).reshape(64, 128)[:n, :rec.d_k].astype(np.float64)
    if rec.scanned:
        out["U"] = np.ctypeslib.as_array(rec.U).reshape(64, 128)[:n, :rec.d_v].astype(np.float64)
    return out


def _check(status: int):
    if status != GDN_OK:
        raise GdnError(status, lib.gdn_last_error().decode())


def _code(dtype: torch.dtype, what: str) -> int:
    if dtype == torch.bfloat16:
        return GDN_BF16
    if dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"{what} dtype must be float32 or bfloat16, got {dtype}")


def conv_state_size(H_k: int, H_v: int, d_k: int, d_v: int) -> int:
    """fp32 values of convolution state at the start of each slot row."""
    return (D_CONV - 1) * (2 * H_k * d_k + H_v * d_v)


def make_dims(H_k: int, H_v: int, d_k: int, d_v: int, dtype: torch.dtype,
              out_dtype: torch.dtype = torch.float32, scale: float = 0.0,
              eps: float = 1e-6, slot_stride: int = 0, gates=None, conv_w=None,
              z=None, norm_w=None) -> Dims:
    """gates: None (g and beta given as the operator takes them) or a pair
    (ssm_a, ssm_dt) of fp32 [H_v] device tensors, with g and beta then holding
    the raw projections a and b (the kernels apply the activations).
    conv_w: [conv_dim, 4] fp32 taps of the fused convolution prologue (q then
    carries the mixed q|k|v rows, k and v are None, state rows start with the
    convolution state).  z, norm_w: the gated RMSNorm epilogue."""
    d = Dims(H_k, H_v, d_k, d_v, _code(dtype, "q/k/v"), _code(out_dtype, "out"),
             slot_stride, scale, eps, GDN_GATES_FINAL, None, None, 0, None, None, None)
    if conv_w is not None:
        _need(conv_w, "conv_w", torch.float32)
        if tuple(conv_w.shape) != (2 * H_k * d_k + H_v * d_v, D_CONV):
            raise ValueError(f"conv_w must be [{2 * H_k * d_k + H_v * d_v}, {D_CONV}]")
        d.d_conv = D_CONV
        d.conv_w = conv_w.data_ptr()
    if z is not None:
        _need(z, "z", dtype)
        if norm_w is None:
            raise ValueError("the epilogue needs norm_w")
        _need(norm_w, "norm_w", torch.float32)
        if norm_w.numel() != d_v or z.shape[-1] != d_v:
            raise ValueError("z and norm_w must end in d_v")
        d.z = z.data_ptr()
        d.norm_w = norm_w.data_ptr()
    if gates is not None:
        ssm_a, ssm_dt = gates
        for t, name in ((ssm_a, "ssm_a"), (ssm_dt, "ssm_dt")):
            _need(t, name, torch.float32)
            if t.numel() != H_v:
                raise ValueError(f"{name} must hold H_v={H_v} values")
        d.gate_mode = GDN_GATES_RAW
        d.ssm_a = ssm_a.data_ptr()
        d.ssm_dt = ssm_dt.data_ptr()
    return d


def _dims_from(q, v, out, scale, eps, state, gates=None, conv=None, z=None, norm_w=None) -> Dims:
    """conv: None, or (conv_w, H_k, d_k) with q the mixed rows [T, conv_dim]
    and v None; the state pools are then [n_slots, row] (convolution state,
    then recurrent state)."""
    stride = 0
    if state is not None and state.dim() in (2, 4):
        stride = state.stride(0)
    if conv is not None:
        conv_w, H_k, d_k = conv
        if v is not None:
            raise ValueError("with the convolution prologue q carries q|k|v: pass k = v = None")
        if q.dim() != 2 or out.dim() != 3:
            raise ValueError("q must be [T, conv_dim], out [T, H_v, d_v]")
        return make_dims(H_k, out.shape[1], d_k, out.shape[2], q.dtype, out.dtype, scale, eps,
                         stride, gates, conv_w, z, norm_w)
    if q.dim() != 3 or v.dim() != 3 or out.shape != v.shape:
        raise ValueError("q must be [T, H_k, d_k], v and out [T, H_v, d_v]")
    return make_dims(q.shape[1], v.shape[1], q.shape[2], v.shape[2], q.dtype, out.dtype,
                     scale, eps, stride, gates, None, z, norm_w)


def _n_slots(*pools) -> int:
    """Slots of the state pools ([n_slots, ...] tensors), for check mode's
    range check of the slot indices (the smallest pool bounds both lists)."""
    n = [t.shape[0] for t in pools if t is not None and t.dim() in (2, 4)]
    return min(n) if n else 0


def _need_qkv(q, k, v, conv):
    dev = q.device
    if conv is None:
        for t, name in ((q, "q"), (k, "k"), (v, "v")):
            _need(t, name, q.dtype, dev)
    else:
        _need(q, "q (mixed rows)", None, dev)
        if k is not None or v is not None:
            raise ValueError("with the convolution prologue k and v must be None")


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype=None, dev=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")


def workspace_size(dims: Dims, n_seqs: int, total_tokens: int) -> int:
    """gdn_prefill_workspace_size: the split-phase calls' workspace (enough for prefill too)."""
    n = ctypes.c_size_t(0)
    _check(lib.gdn_prefill_workspace_size(ctypes.byref(dims), n_seqs, total_tokens, ctypes.byref(n)))
    return n.value


def chunked_workspace_size(dims: Dims, n_seqs: int, total_tokens: int) -> int:
    """gdn_chunked_prefill_workspace_size: the workspace of prefill()."""
    n = ctypes.c_size_t(0)
    _check(lib.gdn_chunked_prefill_workspace_size(ctypes.byref(dims), n_seqs, total_tokens,
                                                  ctypes.byref(n)))
    return n.value


def prefill(q, k, v, g, beta, state_in, state_out, out, cu_seqlens, slot_in, slot_out,
            workspace: Optional[torch.Tensor] = None, *, scale: float = 0.0,
            eps: float = 1e-6, stream=None, gates=None, conv=None, z=None, norm_w=None) -> None:
    """gdn_chunked_prefill on torch tensors (asynchronous on `stream`).
    gates=(ssm_a, ssm_dt): g and beta are the raw projections a, b.
    conv=(conv_w, H_k, d_k): q holds the mixed rows (k = v = None).
    z, norm_w: gated RMSNorm epilogue."""
    dev = q.device
    _need_qkv(q, k, v, conv)
    _need(out, "out", None, dev)
    for t, name in ((g, "g"), (beta, "beta"), (state_out, "state_out")):
        _need(t, name, torch.float32, dev)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, dev)
    for t, name in ((cu_seqlens, "cu_seqlens"), (slot_in, "slot_in"), (slot_out, "slot_out")):
        _need(t, name, torch.int32, dev)
    dims = _dims_from(q, v, out, scale, eps, state_out, gates, conv, z, norm_w)
    dims.n_slots = _n_slots(state_in, state_out)
    n_seqs = slot_out.shape[0]
    T = q.shape[0]
    if workspace is None:
        need = chunked_workspace_size(dims, n_seqs, T)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check(lib.gdn_chunked_prefill(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                   _ptr(beta), _ptr(state_in), _ptr(state_out), _ptr(out),
                                   _ptr(cu_seqlens), _ptr(slot_in), _ptr(slot_out), n_seqs, T,
                                   _ptr(workspace), workspace.numel(), _stream(stream)))


def prefill_noalloc(q, k, v, g, beta, state_in, state_out, out, cu_seqlens, slot_in, slot_out, *,
                    scale: float = 0.0, eps: float = 1e-6, stream=None, gates=None, conv=None,
                    z=None, norm_w=None) -> None:
    """gdn_chunked_prefill_noalloc on torch tensors: prefill() without a
    workspace (the library's own 64 MiB device scratch; nothing is allocated,
    here or in the library)."""
    dev = q.device
    _need_qkv(q, k, v, conv)
    _need(out, "out", None, dev)
    for t, name in ((g, "g"), (beta, "beta"), (state_out, "state_out")):
        _need(t, name, torch.float32, dev)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, dev)
    for t, name in ((cu_seqlens, "cu_seqlens"), (slot_in, "slot_in"), (slot_out, "slot_out")):
        _need(t, name, torch.int32, dev)
    dims = _dims_from(q, v, out, scale, eps, state_out, gates, conv, z, norm_w)
    dims.n_slots = _n_slots(state_in, state_out)
    _check(lib.gdn_chunked_prefill_noalloc(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                           _ptr(beta), _ptr(state_in), _ptr(state_out), _ptr(out),
                                           _ptr(cu_seqlens), _ptr(slot_in), _ptr(slot_out),
                                           slot_out.shape[0], q.shape[0], _stream(stream)))


def _prefill_common(q, k, v, g, beta, state_in, state_out, out, cu_seqlens, slot_in,
                    slot_out, scale, eps):
    dev = q.device
    for t, name in ((q, "q"), (k, "k")):
        _need(t, name, q.dtype, dev)
    if v is not None:
        _need(v, "v", q.dtype, dev)
    if out is not None:
        _need(out, "out", None, dev)
    for t, name in ((g, "g"), (beta, "beta"), (state_out, "state_out"), (state_in, "state_in")):
        if t is not None:
            _need(t, name, torch.float32, dev)
    for t, name in ((cu_seqlens, "cu_seqlens"), (slot_in, "slot_in"), (slot_out, "slot_out")):
        if t is not None:
            _need(t, name, torch.int32, dev)


class PrefillPlan:
    """Dims + workspace for split-phase prefill calls of one batch shape:
    ``prepare(...)`` then ``scan(...)`` (ordered on the caller's streams)."""

    def __init__(self, q, v, out, n_seqs: int, *, state=None, scale: float = 0.0,
                 eps: float = 1e-6, workspace: Optional[torch.Tensor] = None, gates=None,
                 z=None, norm_w=None):
        self.dims = _dims_from(q, v, out, scale, eps, state, gates, None, z, norm_w)
        self.n_seqs = n_seqs
        self.T = q.shape[0]
        need = workspace_size(self.dims, n_seqs, self.T)
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
        elif workspace.numel() < need:
            raise ValueError(f"workspace needs {need} bytes")
        self.workspace = workspace

    def prepare(self, q, k, v, g, beta, cu_seqlens, stream=None):
        _prefill_common(q, k, v, g, beta, None, None, None, cu_seqlens, None, None, 0, 0)
        _check(lib.gdn_prefill_prepare(ctypes.byref(self.dims), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(g), _ptr(beta), _ptr(cu_seqlens), self.n_seqs,
                                       self.T, _ptr(self.workspace), self.workspace.numel(),
                                       _stream(stream)))

    def scan(self, state_in, state_out, out, slot_in, slot_out, stream=None):
        dev = self.workspace.device
        _need(out, "out", None, dev)
        for t, name in ((state_out, "state_out"), (state_in, "state_in")):
            if t is not None:
                _need(t, name, torch.float32, dev)
        for t, name in ((slot_in, "slot_in"), (slot_out, "slot_out")):
            _need(t, name, torch.int32, dev)
        self.dims.n_slots = _n_slots(state_in, state_out)
        _check(lib.gdn_prefill_scan(ctypes.byref(self.dims), _ptr(state_in), _ptr(state_out),
                                    _ptr(out), _ptr(slot_in), _ptr(slot_out), self.n_seqs,
                                    self.T, _ptr(self.workspace), self.workspace.numel(),
                                    _stream(stream)))


def decode_step(q, k, v, g, beta, state_in, state_out, out, slot_in, slot_out, *,
                scale: float = 0.0, eps: float = 1e-6, stream=None, gates=None, conv=None,
                z=None, norm_w=None) -> None:
    """gdn_recurrent_step on torch tensors: one token per sequence."""
    dev = q.device
    _need_qkv(q, k, v, conv)
    _need(out, "out", None, dev)
    for t, name in ((g, "g"), (beta, "beta"), (state_out, "state_out")):
        _need(t, name, torch.float32, dev)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, dev)
    for t, name in ((slot_in, "slot_in"), (slot_out, "slot_out")):
        _need(t, name, torch.int32, dev)
    dims = _dims_from(q, v, out, scale, eps, state_out, gates, conv, z, norm_w)
    dims.n_slots = _n_slots(state_in, state_out)
    _check(lib.gdn_recurrent_step(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                  _ptr(beta), _ptr(state_in), _ptr(state_out), _ptr(out),
                                  _ptr(slot_in), _ptr(slot_out), slot_out.shape[0],
                                  _stream(stream)))


def decode_multi(q, k, v, g, beta, state_in, state_out, out, cu_seqlens, slot_in, slot_out, *,
                 scale: float = 0.0, eps: float = 1e-6, stream=None, gates=None, conv=None,
                 z=None, norm_w=None) -> None:
    """gdn_recurrent_multi on torch tensors: a few tokens per sequence, packed
    by cu_seqlens as for prefill, recurrent form, no workspace."""
    dev = q.device
    _need_qkv(q, k, v, conv)
    _need(out, "out", None, dev)
    for t, name in ((g, "g"), (beta, "beta"), (state_out, "state_out")):
        _need(t, name, torch.float32, dev)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, dev)
    for t, name in ((cu_seqlens, "cu_seqlens"), (slot_in, "slot_in"), (slot_out, "slot_out")):
        _need(t, name, torch.int32, dev)
    dims = _dims_from(q, v, out, scale, eps, state_out, gates, conv, z, norm_w)
    dims.n_slots = _n_slots(state_in, state_out)
    _check(lib.gdn_recurrent_multi(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                   _ptr(beta), _ptr(state_in), _ptr(state_out), _ptr(out),
                                   _ptr(cu_seqlens), _ptr(slot_in), _ptr(slot_out),
                                   slot_out.shape[0], q.shape[0], _stream(stream)))
