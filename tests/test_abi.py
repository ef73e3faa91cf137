"""CPU checks of the C ABI: the library loads, exports every declared symbol,
and its host-side validation rejects bad arguments before touching the GPU.

Every call here fails validation (or is a B = 0 no-op), so no HIP work is ever
enqueued; the pointers are host addresses that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import gated_deltanet_sequence_amd as gdn
from gated_deltanet_sequence_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE, ERR_ALIAS = 0, -1, -2, -3, -4, -5, -6


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gdn\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ["gdn_chunk_fwd", "gdn_chunk_fwd_timed", "gdn_recurrent_step",
                     "gdn_chunk_fwd_workspace_bytes", "gdn_status_str", "gdn_last_error"]:
        assert required in names


def test_library_resolves_all_symbols_at_load():
    # RTLD_NOW: every undefined symbol (e.g. a kernel launch stub the host pass
    # failed to emit) must resolve when the library is loaded
    ctypes.CDLL(binding.LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(binding.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_status_strings():
    L = gdn.lib()
    for code, name in [(0, "GDN_OK"), (-1, "GDN_ERR_NULL"), (-2, "GDN_ERR_SHAPE"),
                       (-3, "GDN_ERR_UNSUPPORTED"), (-4, "GDN_ERR_ALIGN"), (-5, "GDN_ERR_WORKSPACE"),
                       (-6, "GDN_ERR_ALIAS"), (-7, "GDN_ERR_HIP")]:
        assert L.gdn_status_str(code).decode() == name
    assert L.gdn_status_str(99).decode() == "GDN_ERR_UNKNOWN"


class Buf:
    """Host buffers standing in for device pointers (validation only reads addresses)."""

    def __init__(self):
        self._keep = []

    def __call__(self, nbytes, offset=0):
        b = ctypes.create_string_buffer(nbytes + 512)
        self._keep.append(b)
        base = (ctypes.addressof(b) + 255) & ~255
        return base + offset


def dims(**kw):
    d = dict(B=1, T=128, Hk=2, Hv=4, Dk=64, Dv=64, dtype=binding.GDN_BF16, scale=1.0, chunk=64)
    d.update(kw)
    return binding.make_dims(d["B"], d["T"], d["Hk"], d["Hv"], d["Dk"], d["Dv"], d["dtype"],
                             d["scale"], d["chunk"])


def prefill_args(buf, d, **override):
    es = 4 if d.dtype == binding.GDN_F32 else 2
    B, T, Hk, Hv, Dk, Dv = d.B, d.T, d.Hk, d.Hv, d.Dk, d.Dv
    args = dict(
        q=buf(B * T * Hk * Dk * es), k=buf(B * T * Hk * Dk * es), v=buf(B * T * Hv * Dv * es),
        a=buf(B * T * Hv * 4), b=buf(B * T * Hv * 4), A_log=buf(Hv * 4), dt_bias=buf(Hv * 4),
        S0=None, out=buf(B * T * Hv * Dv * es), ST=buf(B * Hv * Dk * Dv * 4))
    ws = binding.lib().gdn_chunk_fwd_workspace_bytes(ctypes.byref(d))
    args["ws"] = buf(ws)
    args["ws_bytes"] = ws
    args.update(override)
    return args


def call_prefill(d, a):
    L = binding.lib()
    return L.gdn_chunk_fwd(ctypes.byref(d), a["q"], a["k"], a["v"], a["a"], a["b"], a["A_log"],
                           a["dt_bias"], a["S0"], a["out"], a["ST"], a["ws"], a["ws_bytes"], None)


def last_error():
    return binding.lib().gdn_last_error().decode()


def test_workspace_bytes():
    L = binding.lib()
    d = dims(B=1, T=4096, Hk=16, Hv=64, Dk=128, Dv=128)
    n = L.gdn_chunk_fwd_workspace_bytes(ctypes.byref(d))
    vunits, kunits = 64 * 64, 16 * 64
    # per (value head, chunk): 8 B token records and two 6 KB operand-fragment sets;
    # per (key head, chunk): Q and K tile images (64 x 128 float16 each)
    need = vunits * (64 * 8 + 2 * 6 * 64 * 8 * 2) + kunits * 2 * 64 * 128 * 2
    assert need <= n < need + 8 * 256
    d_bad = dims(Hv=3)
    assert L.gdn_chunk_fwd_workspace_bytes(ctypes.byref(d_bad)) == 0
    assert L.gdn_chunk_fwd_workspace_bytes(None) == 0
    assert L.gdn_chunk_fwd_workspace_bytes(ctypes.byref(dims(T=0))) == 0
    # float32 operands double the fragment storage
    n32 = L.gdn_chunk_fwd_workspace_bytes(ctypes.byref(dims(B=1, T=4096, Hk=16, Hv=64, Dk=128,
                                                            Dv=128, dtype=binding.GDN_F32)))
    assert n32 > n


@pytest.mark.parametrize("kw,code,needle", [
    (dict(Hv=3), ERR_SHAPE, "multiple"),
    (dict(B=-1), ERR_SHAPE, "B"),
    (dict(T=-5), ERR_SHAPE, "T"),
    (dict(Hk=0), ERR_SHAPE, "Hk"),
    (dict(Dk=96), ERR_UNSUPPORTED, "Dk"),
    (dict(Dv=256), ERR_UNSUPPORTED, "Dv"),
    (dict(chunk=32), ERR_UNSUPPORTED, "chunk"),
    (dict(dtype=7), ERR_UNSUPPORTED, "dtype"),
    (dict(scale=float("nan")), ERR_SHAPE, "scale"),
    # launch-grid and addressing limits
    (dict(B=70000), ERR_SHAPE, "grid limit"),
    (dict(Hk=70000, Hv=70000), ERR_SHAPE, "grid limit"),
    (dict(B=65535, Hk=16, Hv=65520), ERR_SHAPE, "too large"),
    (dict(B=1000, Hk=16, Hv=64, T=64 * 40000), ERR_SHAPE, "too large"),
    (dict(Hk=16, Hv=64, Dk=128, Dv=128, T=131072), ERR_UNSUPPORTED, "limit 2^31"),
])
def test_prefill_rejects_bad_dims(kw, code, needle):
    buf = Buf()
    d = dims(**kw)
    args = prefill_args(buf, dims())
    assert call_prefill(d, args) == code
    assert needle in last_error()


def test_prefill_size_limits_are_exact():
    """The longest bfloat16 sequence at 64 value heads of d_v = 128 that one launch addresses
    with 32-bit byte offsets is accepted (a workspace size comes back); one chunk more is not."""
    L = binding.lib()
    big = dict(B=1, Hk=16, Hv=64, Dk=128, Dv=128)
    ok = L.gdn_chunk_fwd_workspace_bytes(ctypes.byref(dims(T=131072 - 64, **big)))
    assert ok > 0
    assert L.gdn_chunk_fwd_workspace_bytes(ctypes.byref(dims(T=131072 - 63, **big))) == 0
    # float32 inputs halve the token limit
    assert L.gdn_chunk_fwd_workspace_bytes(ctypes.byref(dims(T=65536 - 64, dtype=binding.GDN_F32, **big))) > 0
    assert L.gdn_chunk_fwd_workspace_bytes(ctypes.byref(dims(T=65536 - 63, dtype=binding.GDN_F32, **big))) == 0


def test_prefill_rejects_null_dims():
    L = binding.lib()
    assert L.gdn_chunk_fwd(None, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, None) == ERR_NULL


@pytest.mark.parametrize("name", ["q", "k", "v", "a", "b", "A_log", "dt_bias", "out"])
def test_prefill_rejects_null_pointer(name):
    buf = Buf()
    d = dims()
    args = prefill_args(buf, d, **{name: None})
    assert call_prefill(d, args) == ERR_NULL
    assert name in last_error()


@pytest.mark.parametrize("name", ["q", "v", "out", "ST"])
def test_prefill_rejects_misaligned(name):
    buf = Buf()
    d = dims()
    args = prefill_args(buf, d)
    args[name] = args[name] + 8
    assert call_prefill(d, args) == ERR_ALIGN


def test_prefill_workspace_checks():
    buf = Buf()
    d = dims()
    args = prefill_args(buf, d, ws=None)
    assert call_prefill(d, args) == ERR_WORKSPACE
    args = prefill_args(buf, d)
    args["ws_bytes"] -= 1
    assert call_prefill(d, args) == ERR_WORKSPACE
    args = prefill_args(buf, d)
    args["ws"] += 16
    assert call_prefill(d, args) == ERR_ALIGN


def test_prefill_rejects_aliasing():
    buf = Buf()
    d = dims()
    a = prefill_args(buf, d)
    a["out"] = a["v"]
    assert call_prefill(d, a) == ERR_ALIAS and "out overlaps v" in last_error()
    a = prefill_args(buf, d)
    a["ST"] = a["q"]
    assert call_prefill(d, a) == ERR_ALIAS
    # final_state may equal initial_state, but must not partly overlap it
    a = prefill_args(buf, d)
    s0 = buf(d.B * d.Hv * d.Dk * d.Dv * 4 + 64)
    a["S0"] = s0
    a["ST"] = s0 + 16
    assert call_prefill(d, a) == ERR_ALIAS and "partly" in last_error()
    a = prefill_args(buf, d)
    a["ws"] = a["q"]
    assert call_prefill(d, a) == ERR_ALIAS


def test_prefill_zero_batch_is_a_noop():
    buf = Buf()
    d = dims(B=0)
    a = prefill_args(buf, d, q=None, k=None, v=None, a=None, b=None, out=None, ST=None, ws=None)
    assert call_prefill(d, a) == OK


def test_noalloc_rejects_dims_beyond_its_scratch():
    """gdn_chunk_fwd_noalloc checks the workspace its dims need against its fixed device scratch
    before any HIP call: beyond it, GDN_ERR_WORKSPACE with a message naming both sizes."""
    L = binding.lib()
    buf = Buf()
    limit = binding.NOALLOC_MAX_WORKSPACE_BYTES
    d = dims(B=1, T=8192, Hk=16, Hv=64, Dk=128, Dv=128)
    need = L.gdn_chunk_fwd_workspace_bytes(ctypes.byref(d))
    assert need > limit
    a = prefill_args(buf, dims())  # pointers are never dereferenced: the size check comes first
    st = L.gdn_chunk_fwd_noalloc(ctypes.byref(d), a["q"], a["k"], a["v"], a["a"], a["b"], a["A_log"],
                                 a["dt_bias"], a["S0"], a["out"], a["ST"], None)
    assert st == ERR_WORKSPACE
    assert str(need) in last_error() and str(limit) in last_error()
    # the limit stated in include/gdn.h: 99 chunks of one sequence fit at this head configuration,
    # 100 do not
    d100 = dims(B=1, T=6400, Hk=16, Hv=64, Dk=128, Dv=128)
    assert L.gdn_chunk_fwd_workspace_bytes(ctypes.byref(d100)) > limit
    d99 = dims(B=1, T=6336, Hk=16, Hv=64, Dk=128, Dv=128)
    assert L.gdn_chunk_fwd_workspace_bytes(ctypes.byref(d99)) <= limit
    # invalid dims are reported as such first
    st = L.gdn_chunk_fwd_noalloc(ctypes.byref(dims(Dk=96)), a["q"], a["k"], a["v"], a["a"], a["b"],
                                 a["A_log"], a["dt_bias"], a["S0"], a["out"], a["ST"], None)
    assert st == ERR_UNSUPPORTED


def step_args(buf, d, **override):
    es = 4 if d.dtype == binding.GDN_F32 else 2
    B, Hk, Hv, Dk, Dv = d.B, d.Hk, d.Hv, d.Dk, d.Dv
    args = dict(q=buf(B * Hk * Dk * es), k=buf(B * Hk * Dk * es), v=buf(B * Hv * Dv * es),
                a=buf(B * Hv * 4), b=buf(B * Hv * 4), A_log=buf(Hv * 4), dt_bias=buf(Hv * 4),
                S=buf(B * Hv * Dk * Dv * 4), out=buf(B * Hv * Dv * es))
    args.update(override)
    return args


def call_step(d, a):
    return binding.lib().gdn_recurrent_step(ctypes.byref(d), a["q"], a["k"], a["v"], a["a"], a["b"],
                                            a["A_log"], a["dt_bias"], a["S"], a["out"], None)


def test_step_validation():
    buf = Buf()
    d = dims(B=4)
    assert call_step(dims(B=4, Hv=5), step_args(buf, d)) == ERR_SHAPE
    assert call_step(dims(B=4, Dk=32), step_args(buf, d)) == ERR_UNSUPPORTED
    assert call_step(d, step_args(buf, d, S=None)) == ERR_NULL
    a = step_args(buf, d)
    a["out"] = a["S"]
    assert call_step(d, a) == ERR_ALIAS
    a = step_args(buf, d)
    a["S"] += 4
    assert call_step(d, a) == ERR_ALIGN
    # chunk is ignored by the step: 32 is fine there (fails later only on Hv)
    assert call_step(dims(B=4, chunk=32, Hv=5), step_args(buf, d)) == ERR_SHAPE
    assert call_step(dims(B=0), step_args(buf, dims(B=0))) == OK


def test_binding_rejects_missing_library(tmp_path, monkeypatch):
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        binding.lib()


# ---- Gated DeltaNet-2 prefill (gdn2_chunk_fwd) ----

def gdn2_args(buf, d, **override):
    B, T, Hk, Hv, Dk, Dv = d.B, d.T, d.Hk, d.Hv, d.Dk, d.Dv
    args = dict(
        q=buf(B * T * Hk * Dk * 2), k=buf(B * T * Hk * Dk * 2), v=buf(B * T * Hv * Dv * 2),
        a=buf(B * T * Hv * Dk * 2), A_log=buf(Hv * Dk * 4), erase=buf(B * T * Hv * Dk * 2),
        write=buf(B * T * Hv * Dv * 2), S0=None, out=buf(B * T * Hv * Dv * 2),
        ST=buf(B * Hv * Dk * Dv * 4))
    ws = binding.lib().gdn2_chunk_fwd_workspace_bytes(ctypes.byref(d))
    args["ws"] = buf(ws)
    args["ws_bytes"] = ws
    args.update(override)
    return args


def call_gdn2(d, a):
    return binding.lib().gdn2_chunk_fwd(ctypes.byref(d), a["q"], a["k"], a["v"], a["a"], a["A_log"],
                                        a["erase"], a["write"], a["S0"], a["out"], a["ST"], a["ws"],
                                        a["ws_bytes"], None)


def test_gdn2_declared():
    assert {"gdn2_chunk_fwd", "gdn2_chunk_fwd_workspace_bytes"} <= set(declared_functions())


def test_gdn2_workspace_bytes():
    L = binding.lib()
    d = dims(B=1, T=8192, Hk=16, Hv=64, Dk=128, Dv=128)
    n = L.gdn2_chunk_fwd_workspace_bytes(ctypes.byref(d))
    units = 64 * 128  # (value head, chunk) pairs
    # per unit: three 64 x 128 float16 images (Et, Kh, Q~), two 6 KB fragment sets and the
    # chunk-end decay per key channel (the bfloat16 scan forms Z = sigmoid(write) v itself)
    need = units * (3 * 64 * 128 * 2 + 2 * 6 * 64 * 8 * 2 + 128 * 4)
    assert need <= n < need + 8 * 256
    # float32: the same arrays in float32, plus the 128 x 64 float32 image of Kh^T per unit
    n32 = L.gdn2_chunk_fwd_workspace_bytes(ctypes.byref(dims(B=1, T=8192, Hk=16, Hv=64, Dk=128, Dv=128,
                                                             dtype=binding.GDN_F32)))
    need32 = units * (4 * 64 * 128 * 4 + 2 * 6 * 64 * 8 * 4 + 128 * 4) + 8192 * 64 * 128 * 4
    assert need32 <= n32 < need32 + 9 * 256
    assert L.gdn2_chunk_fwd_workspace_bytes(ctypes.byref(dims(Hv=3))) == 0
    assert L.gdn2_chunk_fwd_workspace_bytes(ctypes.byref(dims(T=0))) == 0
    assert L.gdn2_chunk_fwd_workspace_bytes(None) == 0


def test_gdn2_float32_checks_its_own_workspace_size():
    """A float32 call needs the float32 workspace: the bfloat16 size is refused before
    anything is enqueued."""
    buf = Buf()
    a = gdn2_args(buf, dims())
    d32 = dims(dtype=binding.GDN_F32)
    need32 = binding.lib().gdn2_chunk_fwd_workspace_bytes(ctypes.byref(d32))
    assert need32 > a["ws_bytes"]
    assert call_gdn2(d32, a) == ERR_WORKSPACE
    assert "needed" in last_error()


@pytest.mark.parametrize("kw,code", [(dict(Hv=3), ERR_SHAPE), (dict(Dk=96), ERR_UNSUPPORTED),
                                     (dict(chunk=32), ERR_UNSUPPORTED), (dict(T=-1), ERR_SHAPE)])
def test_gdn2_rejects_bad_dims(kw, code):
    buf = Buf()
    assert call_gdn2(dims(**kw), gdn2_args(buf, dims())) == code


@pytest.mark.parametrize("name", ["q", "k", "v", "a", "A_log", "erase", "write", "out"])
def test_gdn2_rejects_null_pointer(name):
    buf = Buf()
    d = dims()
    assert call_gdn2(d, gdn2_args(buf, d, **{name: None})) == ERR_NULL
    assert name in last_error()


@pytest.mark.parametrize("name", ["a", "erase", "write", "ST"])
def test_gdn2_rejects_misaligned(name):
    buf = Buf()
    d = dims()
    a = gdn2_args(buf, d)
    a[name] += 8
    assert call_gdn2(d, a) == ERR_ALIGN


def test_gdn2_workspace_and_alias_checks():
    buf = Buf()
    d = dims()
    assert call_gdn2(d, gdn2_args(buf, d, ws=None)) == ERR_WORKSPACE
    a = gdn2_args(buf, d)
    a["ws_bytes"] -= 1
    assert call_gdn2(d, a) == ERR_WORKSPACE
    a = gdn2_args(buf, d)
    a["out"] = a["write"]
    assert call_gdn2(d, a) == ERR_ALIAS and "out overlaps write" in last_error()
    a = gdn2_args(buf, d)
    a["ST"] = a["erase"]
    assert call_gdn2(d, a) == ERR_ALIAS
    a = gdn2_args(buf, d)
    s0 = buf(d.B * d.Hv * d.Dk * d.Dv * 4 + 64)
    a["S0"], a["ST"] = s0, s0 + 16
    assert call_gdn2(d, a) == ERR_ALIAS and "partly" in last_error()
    a = gdn2_args(buf, d)
    a["ws"] = a["a"]
    assert call_gdn2(d, a) == ERR_ALIAS


def test_gdn2_zero_batch_is_a_noop():
    buf = Buf()
    d = dims(B=0)
    a = gdn2_args(buf, d, q=None, k=None, v=None, a=None, erase=None, write=None, out=None, ST=None,
                  ws=None)
    assert call_gdn2(d, a) == OK


# ---- Gated DeltaNet-2 backward (gdn2_chunk_bwd) ----

def bwd2_args(buf, d, **override):
    B, T, Hk, Hv, Dk, Dv = d.B, d.T, d.Hk, d.Hv, d.Dk, d.Dv
    args = dict(
        q=buf(B * T * Hk * Dk * 2), k=buf(B * T * Hk * Dk * 2), v=buf(B * T * Hv * Dv * 2),
        a=buf(B * T * Hv * Dk * 2), A_log=buf(Hv * Dk * 4), erase=buf(B * T * Hv * Dk * 2),
        write=buf(B * T * Hv * Dv * 2), S0=None, dout=buf(B * T * Hv * Dv * 2), dST=None,
        dq=buf(B * T * Hk * Dk * 4), dk=buf(B * T * Hk * Dk * 4), dv=buf(B * T * Hv * Dv * 4),
        da=buf(B * T * Hv * Dk * 4), derase=buf(B * T * Hv * Dk * 4), dwrite=buf(B * T * Hv * Dv * 4),
        dAl=buf(Hv * Dk * 4), dS0=buf(B * Hv * Dk * Dv * 4))
    ws = binding.lib().gdn2_chunk_bwd_workspace_bytes(ctypes.byref(d))
    args["ws"] = buf(ws)
    args["ws_bytes"] = ws
    args.update(override)
    return args


def call_bwd2(d, a):
    return binding.lib().gdn2_chunk_bwd(
        ctypes.byref(d), a["q"], a["k"], a["v"], a["a"], a["A_log"], a["erase"], a["write"], a["S0"],
        a["dout"], a["dST"], a["dq"], a["dk"], a["dv"], a["da"], a["derase"], a["dwrite"], a["dAl"],
        a["dS0"], a["ws"], a["ws_bytes"], None)


def test_bwd2_declared():
    assert {"gdn2_chunk_bwd", "gdn2_chunk_bwd_timed", "gdn2_chunk_bwd_workspace_bytes"} <= set(declared_functions())


def test_bwd2_workspace_bytes():
    L = binding.lib()
    n = L.gdn2_chunk_bwd_workspace_bytes(ctypes.byref(dims(B=1, T=8192, Hk=16, Hv=64, Dk=128, Dv=128)))
    units = 64 * 128
    # per unit, float32, with the gradients written into the space of buffers already read
    # for the last time: A | dM, A_qk | dA_qk (64 x 64); Et | dEt, Qt | dQt, Kh | dKh (64 x Dk);
    # R, U | dA_log part, dU, dR (64 x Dv); S_n | dq, dS_{n+1} | dk (Dk x Dv; dq and dk per
    # value head [B,T,Hv,Dk] fit there); e^{G_C} | its gradient (Dk)
    need = units * 4 * (2 * 64 * 64 + 3 * 64 * 128 + 4 * 64 * 128 + 2 * 128 * 128 + 128)
    assert need <= n < need + 12 * 256
    assert n < 3.3e9
    # float32 inputs: the same float32 workspace
    assert L.gdn2_chunk_bwd_workspace_bytes(ctypes.byref(dims(dtype=binding.GDN_F32))) == \
        L.gdn2_chunk_bwd_workspace_bytes(ctypes.byref(dims()))
    assert L.gdn2_chunk_bwd_workspace_bytes(ctypes.byref(dims(T=0))) == 0
    assert L.gdn2_chunk_bwd_workspace_bytes(None) == 0


def test_bwd2_validation():
    buf = Buf()
    d = dims()
    assert call_bwd2(dims(Hv=3), bwd2_args(buf, d)) == ERR_SHAPE
    assert call_bwd2(dims(Dk=96), bwd2_args(buf, d)) == ERR_UNSUPPORTED
    for name in ["q", "k", "v", "a", "A_log", "erase", "write", "dout", "dq", "dk", "dv", "da", "derase",
                 "dwrite", "dAl"]:
        assert call_bwd2(d, bwd2_args(buf, d, **{name: None})) == ERR_NULL, name
    for name in ["dq", "da", "dwrite", "dS0"]:
        a = bwd2_args(buf, d)
        a[name] += 8
        assert call_bwd2(d, a) == ERR_ALIGN, name
    assert call_bwd2(d, bwd2_args(buf, d, ws=None)) == ERR_WORKSPACE
    a = bwd2_args(buf, d)
    a["ws_bytes"] -= 1
    assert call_bwd2(d, a) == ERR_WORKSPACE
    a = bwd2_args(buf, d)
    a["dv"] = a["v"]
    assert call_bwd2(d, a) == ERR_ALIAS and "dv overlaps v" in last_error()
    a = bwd2_args(buf, d)
    a["da"] = a["derase"]
    assert call_bwd2(d, a) == ERR_ALIAS
    a = bwd2_args(buf, d)
    a["dS0"] = a["ws"]
    assert call_bwd2(d, a) == ERR_ALIAS
    # B = 0: the per-token tensors are empty (their pointers unused), but dA_log [Hv,Dk] is
    # still written (zeros), so it must be given; the zeroing itself is a GPU test
    d0 = dims(B=0)
    assert call_bwd2(d0, bwd2_args(buf, d0, q=None, k=None, v=None, a=None, erase=None, write=None,
                                   dout=None, dq=None, dk=None, dv=None, da=None, derase=None,
                                   dwrite=None, dS0=None, ws=None, dAl=None)) == ERR_NULL


# ---- Gated DeltaNet-2 decode step (gdn2_recurrent_step) ----

def step2_args(buf, d, **override):
    es = 4 if d.dtype == binding.GDN_F32 else 2
    B, Hk, Hv, Dk, Dv = d.B, d.Hk, d.Hv, d.Dk, d.Dv
    args = dict(q=buf(B * Hk * Dk * es), k=buf(B * Hk * Dk * es), v=buf(B * Hv * Dv * es),
                a=buf(B * Hv * Dk * es), A_log=buf(Hv * Dk * 4), erase=buf(B * Hv * Dk * es),
                write=buf(B * Hv * Dv * es), S=buf(B * Hv * Dk * Dv * 4), out=buf(B * Hv * Dv * es))
    args.update(override)
    return args


def call_step2(d, a):
    return binding.lib().gdn2_recurrent_step(ctypes.byref(d), a["q"], a["k"], a["v"], a["a"], a["A_log"],
                                             a["erase"], a["write"], a["S"], a["out"], None)


def test_gdn2_step_declared():
    assert "gdn2_recurrent_step" in declared_functions()


@pytest.mark.parametrize("name", ["q", "k", "v", "a", "A_log", "erase", "write", "S", "out"])
def test_gdn2_step_rejects_null(name):
    buf = Buf()
    d = dims(B=4)
    assert call_step2(d, step2_args(buf, d, **{name: None})) == ERR_NULL


def test_gdn2_step_validation():
    buf = Buf()
    d = dims(B=4)
    assert call_step2(dims(B=4, Hv=5), step2_args(buf, d)) == ERR_SHAPE
    assert call_step2(dims(B=4, Dv=32), step2_args(buf, d)) == ERR_UNSUPPORTED
    for name in ("write", "erase", "S"):
        a = step2_args(buf, d)
        a[name] += 8
        assert call_step2(d, a) == ERR_ALIGN, name
    a = step2_args(buf, d)
    a["out"] = a["write"]
    assert call_step2(d, a) == ERR_ALIAS and "out overlaps write" in last_error()
    a = step2_args(buf, d)
    a["S"] = a["a"]
    assert call_step2(d, a) == ERR_ALIAS
    # fp32 is accepted by the step (validation passes up to the B = 0 no-op)
    d32 = dims(B=0, dtype=binding.GDN_F32)
    assert call_step2(d32, step2_args(buf, d32)) == OK
    assert call_step2(dims(B=0), step2_args(buf, dims(B=0))) == OK


# ---- gated RMS normalisation (gdn_gated_rmsnorm) ----

def call_norm(rows, d, dtype, x, z, w, eps=1e-6, gate=0, out=None):
    return binding.lib().gdn_gated_rmsnorm(rows, d, dtype, x, z, w, eps, gate, out, None)


def test_gated_rmsnorm_validation():
    buf = Buf()
    rows, d = 10, 128
    x, z, w, o = buf(rows * d * 2), buf(rows * d * 2), buf(d * 4), buf(rows * d * 2)
    bf = binding.GDN_BF16
    assert "gdn_gated_rmsnorm" in declared_functions()
    assert call_norm(-1, d, bf, x, z, w, out=o) == ERR_SHAPE
    assert call_norm(rows, 96, bf, x, z, w, out=o) == ERR_UNSUPPORTED
    assert call_norm(rows, d, 5, x, z, w, out=o) == ERR_UNSUPPORTED
    assert call_norm(rows, d, bf, x, z, w, gate=2, out=o) == ERR_UNSUPPORTED
    assert call_norm(rows, d, bf, x, z, w, eps=-1.0, out=o) == ERR_SHAPE
    assert call_norm(rows, d, bf, x, z, w, eps=float("inf"), out=o) == ERR_SHAPE
    assert call_norm(rows, d, bf, None, z, w, out=o) == ERR_NULL
    assert call_norm(rows, d, bf, x, z, None, out=o) == ERR_NULL
    assert call_norm(rows, d, bf, x + 8, z, w, out=o) == ERR_ALIGN
    assert call_norm(rows, d, bf, x, z, w, out=z) == ERR_ALIAS
    assert call_norm(rows, d, bf, x, z, w, out=x + 16) == ERR_ALIAS and "partly" in last_error()
    assert call_norm(0, d, bf, None, None, None, out=None) == OK


# ---- causal conv1d prologue (gdn_causal_conv1d) ----

def conv_args(buf, d, K=4):
    es = 4 if d.dtype == binding.GDN_F32 else 2
    qk, vw = d.Hk * d.Dk, d.Hv * d.Dv
    C = 2 * qk + vw
    return dict(x=buf(d.B * d.T * C * es), w=buf(C * K * 4), b=buf(C * 4), s=buf(d.B * (K - 1) * C * es),
                so=buf(d.B * (K - 1) * C * es), q=buf(d.B * d.T * qk * es), k=buf(d.B * d.T * qk * es),
                v=buf(d.B * d.T * vw * es))


def call_conv(d, a, K=4, act=1):
    return binding.lib().gdn_causal_conv1d(ctypes.byref(d), K, a["x"], a["w"], a["b"], a["s"], a["so"], act,
                                           a["q"], a["k"], a["v"], None)


def test_causal_conv1d_validation():
    buf = Buf()
    d = dims(B=2, T=20)
    assert "gdn_causal_conv1d" in declared_functions()
    assert call_conv(d, conv_args(buf, d), K=3) == ERR_UNSUPPORTED
    assert call_conv(d, conv_args(buf, d), act=7) == ERR_UNSUPPORTED
    assert call_conv(dims(B=2, T=-1), conv_args(buf, d)) == ERR_SHAPE
    assert call_conv(dims(B=70000, T=1), conv_args(buf, dims(B=1, T=1))) == ERR_UNSUPPORTED
    for name in ("x", "w", "q", "k", "v"):
        a = conv_args(buf, d)
        a[name] = None
        assert call_conv(d, a) == ERR_NULL, name
    a = conv_args(buf, d)
    a["x"] += 8
    assert call_conv(d, a) == ERR_ALIGN
    a = conv_args(buf, d)
    a["q"] = a["x"]
    assert call_conv(d, a) == ERR_ALIAS
    a = conv_args(buf, d)
    a["v"] = a["k"]
    assert call_conv(d, a) == ERR_ALIAS and "overlaps" in last_error()
    a = conv_args(buf, d)
    a["so"] = a["s"] + 16
    assert call_conv(d, a) == ERR_ALIAS and "partly" in last_error()
    a = conv_args(buf, d)
    a["so"] = a["s"]  # in place: allowed (B = 0 keeps the call host-only)
    d0 = dims(B=0, T=20)
    assert call_conv(d0, conv_args(buf, d0)) == OK
    a0 = conv_args(buf, d0)
    a0["b"] = a0["s"] = a0["so"] = None
    assert call_conv(d0, a0) == OK
