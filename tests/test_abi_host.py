"""The C ABI on the host: the library loads, exports every declared symbol,
and rejects bad arguments before anything is enqueued (no GPU needed: every
call here fails validation before it reaches the HIP runtime)."""
import ctypes
import os
import re

import pytest

import gated_deltanet_rule_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(gdn.EXPORTED)
    raw = ctypes.CDLL(gdn.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_version_and_status_strings():
    assert gdn.version() == 6
    for st in range(5):
        assert gdn.lib.gdn_status_string(st)
    assert gdn.lib.gdn_status_string(99) == b"unknown status"


def _dims(**kw):
    base = dict(H_k=16, H_v=32, d_k=128, d_v=128, dtype=gdn.GDN_BF16, out_dtype=0,
                slot_stride=0, scale=0.0, eps=1e-6)
    base.update(kw)
    d = gdn.Dims()
    for k, v in base.items():
        setattr(d, k, v)
    return d


def test_workspace_size_grows_with_tokens_and_is_aligned():
    a = gdn.workspace_size(_dims(), 1, 4096)
    b = gdn.workspace_size(_dims(), 1, 8192)
    c = gdn.workspace_size(_dims(), 8, 4096)
    assert 0 < a < b and a < c
    # per (64-token chunk, value head): W, T', P fragments + scalars
    # 64 more chunks x (32 value-head blocks: W 16 + P 2x8 + scalars 1 + U0 32 KiB,
    #                   16 key-head blocks: q 16 + k^T 16 KiB)
    blocks = 64 * (32 * (16 + 16 + 1 + 32) + 16 * 32) * 1024
    assert 0 <= (b - a) - blocks <= 64 * 16 + 256  # + their chunk-table entries
    f = gdn.workspace_size(_dims(dtype=gdn.GDN_F32), 1, 4096)
    assert f > a


def test_chunked_workspace_holds_one_range():
    """gdn_chunked_prefill's workspace holds the factors of one chunk range
    (at these heads: every chunk up to 212 MiB of factors, else 64 chunks)
    plus, when the batch runs as several ranges, two carry states; the
    split-phase layout holds a slot for each of the batch's at most
    T/64 + n_seqs chunks and no carry state.  The rest of the two layouts is
    the same."""
    d = _dims()
    slot = (32 * (16 + 16 + 1 + 32) + 16 * 32) * 1024     # one chunk's factors, all heads
    carry = 2 * 32 * 128 * 128 * 4                        # two H_v x d_k x d_v fp32 states
    for n, T, held in ((1, 4096, 64), (1, 4160, 65), (1, 8229, 64), (1, 65536, 64),
                       (8, 12221, 64), (8, 512, 16)):
        full = gdn.workspace_size(d, n, T)
        part = gdn.chunked_workspace_size(d, n, T)
        bound = (T + 63) // 64 + n
        chunks = (T + 63) // 64 if n == 1 else bound
        if n > 1 and bound * slot <= 212 << 20:
            held = bound                                  # one range over the bound
        ranges = held < chunks
        assert full - part == (bound - held) * slot - (carry if ranges else 0), (n, T)
    assert gdn.workspace_size(d, 1, 65536) > 2.7e9
    assert gdn.chunked_workspace_size(d, 1, 65536) < 0.18e9


@pytest.mark.parametrize("kw,status", [
    (dict(H_k=0), 1), (dict(H_v=-1), 1), (dict(H_v=24, H_k=16), 2),
    (dict(d_k=96), 2), (dict(d_v=256), 2), (dict(dtype=7), 2), (dict(out_dtype=3), 2),
    (dict(slot_stride=100), 1), (dict(slot_stride=32 * 128 * 128 + 2), 1),
    (dict(eps=-1.0), 1), (dict(scale=float("nan")), 1),
    (dict(gate_mode=2), 1), (dict(gate_mode=-1), 1),
    (dict(gate_mode=gdn.GDN_GATES_RAW), 1),                       # no ssm_a / ssm_dt
    (dict(gate_mode=gdn.GDN_GATES_RAW, ssm_a=0x1000), 1),         # ssm_dt missing
    (dict(gate_mode=gdn.GDN_GATES_RAW, ssm_a=0x1002, ssm_dt=0x2000), 1),  # misaligned
    (dict(d_conv=3, conv_w=0x1000), 2), (dict(d_conv=-4, conv_w=0x1000), 2),
    (dict(d_conv=4), 1),                                          # no taps
    (dict(d_conv=4, conv_w=0x1004), 1),                           # misaligned taps
    (dict(z=0x1000), 1),                                          # no norm weight
    (dict(z=0x1008, norm_w=0x2000), 1), (dict(z=0x1000, norm_w=0x2004), 1),
    # with the prologue a slot row also holds 3 * conv_dim convolution state
    (dict(d_conv=4, conv_w=0x1000, slot_stride=32 * 128 * 128), 1),
    (dict(n_slots=-1), 1),
])
def test_bad_dims_rejected(kw, status):
    n = ctypes.c_size_t(0)
    st = gdn.lib.gdn_prefill_workspace_size(ctypes.byref(_dims(**kw)), 1, 64, ctypes.byref(n))
    assert st == status
    assert gdn.lib.gdn_last_error()


def test_raw_gates_accepted_by_sizing():
    # With both pointers present and aligned the dims are valid; the sizing
    # call never dereferences them.
    n = ctypes.c_size_t(0)
    d = _dims(gate_mode=gdn.GDN_GATES_RAW, ssm_a=0x1000, ssm_dt=0x2000)
    assert gdn.lib.gdn_prefill_workspace_size(ctypes.byref(d), 1, 64, ctypes.byref(n)) == 0
    m = ctypes.c_size_t(0)
    assert gdn.lib.gdn_prefill_workspace_size(ctypes.byref(_dims()), 1, 64, ctypes.byref(m)) == 0
    assert n.value == m.value


def test_conv_rows_grow_the_slot():
    n = ctypes.c_size_t(0)
    C = 2 * 16 * 128 + 32 * 128
    ok = _dims(d_conv=4, conv_w=0x1000, slot_stride=32 * 128 * 128 + 3 * C)
    assert gdn.lib.gdn_prefill_workspace_size(ctypes.byref(ok), 1, 64, ctypes.byref(n)) == 0
    assert gdn.conv_state_size(16, 32, 128, 128) == 3 * C


def test_null_dims_and_counts():
    n = ctypes.c_size_t(0)
    assert gdn.lib.gdn_prefill_workspace_size(None, 1, 64, ctypes.byref(n)) == 1
    assert gdn.lib.gdn_prefill_workspace_size(ctypes.byref(_dims()), 0, 64, ctypes.byref(n)) == 1
    assert gdn.lib.gdn_prefill_workspace_size(ctypes.byref(_dims()), 1, -5, ctypes.byref(n)) == 1
    assert gdn.lib.gdn_prefill_workspace_size(ctypes.byref(_dims()), 1, 64, None) == 1


FAKE = 0x7f0000000000  # never dereferenced: every call below fails validation


def _prefill_args(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, state_in=FAKE, state_out=FAKE,
             out=FAKE, cu=FAKE, sin=FAKE, sout=FAKE, n=1, T=64, ws=FAKE, wsb=1 << 40)
    a.update(over)
    return a


def _call_prefill(d, a):
    P = ctypes.c_void_p
    return gdn.lib.gdn_chunked_prefill(
        ctypes.byref(d), P(a["q"]), P(a["k"]), P(a["v"]), P(a["g"]), P(a["beta"]),
        P(a["state_in"]), P(a["state_out"]), P(a["out"]), P(a["cu"]), P(a["sin"]),
        P(a["sout"]), a["n"], a["T"], P(a["ws"]), a["wsb"], None)


@pytest.mark.parametrize("over,status", [
    (dict(q=0), 1), (dict(k=0), 1), (dict(v=0), 1), (dict(g=0), 1), (dict(beta=0), 1),
    (dict(state_out=0), 1), (dict(out=0), 1), (dict(cu=0), 1), (dict(sin=0), 1),
    (dict(sout=0), 1), (dict(q=FAKE + 8), 1), (dict(g=FAKE + 2), 1),
    (dict(state_in=FAKE + 4), 1), (dict(n=0), 1), (dict(T=-1), 1), (dict(T=1 << 33), 1),
    (dict(ws=0), 3), (dict(wsb=1000), 3), (dict(ws=FAKE + 16), 3),
])
def test_prefill_validation(over, status):
    assert _call_prefill(_dims(), _prefill_args(**over)) == status
    assert gdn.lib.gdn_last_error()


def test_split_phase_validation():
    P = ctypes.c_void_p
    d = _dims()
    prep = lambda **o: gdn.lib.gdn_prefill_prepare(
        ctypes.byref(d), P(o.get("q", FAKE)), P(o.get("k", FAKE)), P(o.get("v", FAKE)),
        P(o.get("g", FAKE)), P(o.get("beta", FAKE)), P(o.get("cu", FAKE)), o.get("n", 1),
        o.get("T", 64), P(o.get("ws", FAKE)), o.get("wsb", 1 << 40), None)
    assert prep(q=0) == 1 and prep(v=0) == 1 and prep(cu=0) == 1 and prep(g=FAKE + 1) == 1
    assert prep(n=0) == 1 and prep(wsb=16) == 3 and prep(ws=0) == 3
    scan = lambda **o: gdn.lib.gdn_prefill_scan(
        ctypes.byref(d), P(o.get("si", FAKE)), P(o.get("so", FAKE)), P(o.get("out", FAKE)),
        P(o.get("sin", FAKE)), P(o.get("sout", FAKE)), o.get("n", 1), o.get("T", 64),
        P(o.get("ws", FAKE)), o.get("wsb", 1 << 40), None)
    assert scan(so=0) == 1 and scan(out=FAKE + 4) == 1 and scan(sin=0) == 1
    assert scan(T=-2) == 1 and scan(wsb=16) == 3


def test_decode_validation():
    P = ctypes.c_void_p
    d = _dims()

    def call(**over):
        a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, si=FAKE, so=FAKE, out=FAKE,
                 sin=FAKE, sout=FAKE, n=4)
        a.update(over)
        return gdn.lib.gdn_recurrent_step(ctypes.byref(d), P(a["q"]), P(a["k"]), P(a["v"]),
                                          P(a["g"]), P(a["beta"]), P(a["si"]), P(a["so"]),
                                          P(a["out"]), P(a["sin"]), P(a["sout"]), a["n"], None)
    assert call(q=0) == 1
    assert call(so=0) == 1
    assert call(out=FAKE + 2) == 1
    assert call(n=0) == 1
    assert call(sout=FAKE + 1) == 1
    assert gdn.lib.gdn_recurrent_step(None, *([None] * 10), 1, None) == 1


def test_multi_decode_validation():
    P = ctypes.c_void_p
    d = _dims()

    def call(**over):
        a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, si=FAKE, so=FAKE, out=FAKE,
                 cu=FAKE, sin=FAKE, sout=FAKE, n=4, T=16)
        a.update(over)
        return gdn.lib.gdn_recurrent_multi(
            ctypes.byref(d), P(a["q"]), P(a["k"]), P(a["v"]), P(a["g"]), P(a["beta"]),
            P(a["si"]), P(a["so"]), P(a["out"]), P(a["cu"]), P(a["sin"]), P(a["sout"]),
            a["n"], a["T"], None)
    assert call(q=0) == 1
    assert call(cu=0) == 1
    assert call(so=0) == 1
    assert call(out=FAKE + 2) == 1
    assert call(n=0) == 1
    assert call(T=-1) == 1
    assert call(sout=FAKE + 1) == 1
    assert gdn.lib.gdn_recurrent_multi(None, *([None] * 11), 1, 4, None) == 1



def test_prologue_argument_rules():
    """With d_conv, q carries the mixed rows: k and v must be NULL; the
    split-phase entry points reject the prologue (it reads the slot state)."""
    P = ctypes.c_void_p
    d = _dims(d_conv=4, conv_w=0x1000)
    assert _call_prefill(d, _prefill_args()) == 1            # k, v given
    assert b"NULL" in gdn.lib.gdn_last_error()
    st = gdn.lib.gdn_prefill_prepare(ctypes.byref(d), P(FAKE), None, None, P(FAKE), P(FAKE),
                                     P(FAKE), 1, 64, P(FAKE), 1 << 40, None)
    assert st == 2
    st = gdn.lib.gdn_prefill_scan(ctypes.byref(d), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                                  1, 64, P(FAKE), 1 << 40, None)
    assert st == 2
    st = gdn.lib.gdn_recurrent_step(ctypes.byref(d), P(FAKE), P(FAKE), None, P(FAKE), P(FAKE),
                                    P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 4, None)
    assert st == 1
    st = gdn.lib.gdn_recurrent_multi(ctypes.byref(d), None, None, None, P(FAKE), P(FAKE),
                                     P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 4, 16, None)
    assert st == 1


def test_dims_layout_matches_the_header(tmp_path):
    """The binding's ctypes structure has the C struct's size and field
    offsets (compiled from include/gdn.h with the host compiler)."""
    import subprocess
    fields = [f for f, _ in gdn.Dims._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "gdn.h"\nint main(void){\n'
                   + 'printf("%zu\\n", sizeof(gdn_dims));\n'
                   + "".join(f'printf("%zu\\n", offsetof(gdn_dims, {f}));\n' for f in fields)
                   + "return 0;}\n")
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run(["gcc", "-std=c99", "-I", inc, str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(gdn.Dims)
    for f, off in zip(fields, got[1:]):
        assert getattr(gdn.Dims, f).offset == off, f


def test_debug_record_layout_matches_the_header(tmp_path):
    """gdn_debug_chunk: the binding's structure has the C struct's size and
    field offsets."""
    import subprocess
    fields = [f for f, _ in gdn.DebugChunk._fields_]
    src = tmp_path / "dbg.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "gdn.h"\nint main(void){\n'
                   + 'printf("%zu\\n", sizeof(gdn_debug_chunk));\n'
                   + "".join(f'printf("%zu\\n", offsetof(gdn_debug_chunk, {f}));\n' for f in fields)
                   + "return 0;}\n")
    exe = tmp_path / "dbg"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run(["gcc", "-std=c99", "-I", inc, str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(gdn.DebugChunk)
    for f, off in zip(fields, got[1:]):
        assert getattr(gdn.DebugChunk, f).offset == off, f


def test_debug_dump_without_a_record():
    """No prefill has run with GDN_DEBUG_DUMP in this process: the accessor
    reports it (and a NULL destination) without touching a device."""
    assert gdn.lib.gdn_debug_dump(None) == 1
    rec = gdn.DebugChunk()
    assert gdn.lib.gdn_debug_dump(ctypes.byref(rec)) == 1
    assert "GDN_DEBUG_DUMP" in gdn.lib.gdn_last_error().decode()
