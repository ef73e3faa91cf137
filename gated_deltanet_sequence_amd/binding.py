"""Thin ctypes binding of libgdn.so (include/gdn.h) for torch tensors.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  Torch supplies device memory and the current
stream.  If the library is missing this module raises at load time; there is
no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")

GDN_F32, GDN_BF16 = 0, 1
GDN_CHUNK_FWD_STAGES = 2
STAGE_NAMES = ("chunk_local", "state_scan")
GDN2_CHUNK_BWD_STAGES = 6
BWD2_STAGE_NAMES = ("g2b_prep", "g2b_fwd_scan", "g2b_bwd_scan", "g2b_products", "g2b_local", "g2b_reduce")


class gdn_dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("Hk", ctypes.c_int32),
                ("Hv", ctypes.c_int32), ("Dk", ctypes.c_int32), ("Dv", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


class GDNError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}" if detail else name)
        self.status = status


_lib = None


def lib():
    """Load libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m gated_deltanet_sequence_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, fp, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t
    dims_p = ctypes.POINTER(gdn_dims)
    L.gdn_chunk_fwd_workspace_bytes.restype = sz
    L.gdn_chunk_fwd_workspace_bytes.argtypes = [dims_p]
    L.gdn_chunk_fwd.restype = ctypes.c_int
    L.gdn_chunk_fwd.argtypes = [dims_p, vp, vp, vp, fp, fp, fp, fp, fp, vp, fp, vp, sz, vp]
    L.gdn_chunk_fwd_timed.restype = ctypes.c_int
    L.gdn_chunk_fwd_timed.argtypes = [dims_p, vp, vp, vp, fp, fp, fp, fp, fp, vp, fp, vp, sz, vp,
                                      ctypes.POINTER(ctypes.c_void_p)]
    L.gdn_chunk_fwd_noalloc.restype = ctypes.c_int
    L.gdn_chunk_fwd_noalloc.argtypes = [dims_p, vp, vp, vp, fp, fp, fp, fp, fp, vp, fp, vp]
    L.gdn2_chunk_fwd_workspace_bytes.restype = sz
    L.gdn2_chunk_fwd_workspace_bytes.argtypes = [dims_p]
    L.gdn2_chunk_fwd.restype = ctypes.c_int
    L.gdn2_chunk_fwd.argtypes = [dims_p, vp, vp, vp, vp, fp, vp, vp, fp, vp, fp, vp, sz, vp]
    L.gdn2_chunk_bwd_workspace_bytes.restype = sz
    L.gdn2_chunk_bwd_workspace_bytes.argtypes = [dims_p]
    L.gdn2_chunk_bwd.restype = ctypes.c_int
    L.gdn2_chunk_bwd.argtypes = [dims_p, vp, vp, vp, vp, fp, vp, vp, fp, vp, fp,
                                 fp, fp, fp, fp, fp, fp, fp, fp, vp, sz, vp]
    L.gdn2_chunk_bwd_timed.restype = ctypes.c_int
    L.gdn2_chunk_bwd_timed.argtypes = L.gdn2_chunk_bwd.argtypes + [ctypes.POINTER(ctypes.c_void_p)]
    L.gdn_recurrent_step.restype = ctypes.c_int
    L.gdn_recurrent_step.argtypes = [dims_p, vp, vp, vp, fp, fp, fp, fp, fp, vp, vp]
    L.gdn2_recurrent_step.restype = ctypes.c_int
    L.gdn2_recurrent_step.argtypes = [dims_p, vp, vp, vp, vp, fp, vp, vp, fp, vp, vp]
    L.gdn_gated_rmsnorm.restype = ctypes.c_int
    L.gdn_gated_rmsnorm.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp, vp, fp,
                                    ctypes.c_float, ctypes.c_int32, vp, vp]
    L.gdn_causal_conv1d.restype = ctypes.c_int
    L.gdn_causal_conv1d.argtypes = [dims_p, ctypes.c_int32, vp, fp, fp, vp, vp, ctypes.c_int32, vp, vp, vp, vp]
    L.gdn_status_str.restype = ctypes.c_char_p
    L.gdn_status_str.argtypes = [ctypes.c_int]
    L.gdn_last_error.restype = ctypes.c_char_p
    L.gdn_last_error.argtypes = []
    L.gdn_events_create.restype = ctypes.c_int
    L.gdn_events_create.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_void_p)]
    L.gdn_events_destroy.restype = ctypes.c_int
    L.gdn_events_destroy.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_void_p)]
    L.gdn_event_elapsed_ms.restype = ctypes.c_int
    L.gdn_event_elapsed_ms.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_float)]
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        L = lib()
        raise GDNError(status, L.gdn_status_str(status).decode(), L.gdn_last_error().decode())


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return GDN_F32
    if t == torch.bfloat16:
        return GDN_BF16
    raise TypeError(f"unsupported dtype {t}: float32 or bfloat16")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr() if t.numel() else None


def _validate(dev, specs):
    """Check every (name, tensor, shape, dtype) of specs: a torch tensor of that shape and
    dtype (None: any), contiguous, on the GPU device dev.  A spec whose tensor is None is an
    omitted optional argument and is skipped.  Shapes and dtypes of all tensors are checked
    before any device, so a wrong size is reported as such whatever the device; a host tensor
    (whose address a kernel would fault on) is rejected before anything is enqueued."""
    for name, t, shape, dtype in specs:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (isinstance(dev, torch.device) and dev.type == "cuda"):
        raise ValueError(f"inputs must be GPU tensors (got {dev})")
    for name, t, _, _ in specs:
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _workspace_spec(workspace, need: int):
    """The workspace must hold at least `need` bytes (also checked by the library)."""
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor):
            raise TypeError("workspace must be a torch.Tensor")
        if workspace.numel() * workspace.element_size() < need:
            raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, "
                             f"{need} needed")
    return ("workspace", workspace, None, None)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def make_dims(B, T, Hk, Hv, Dk, Dv, dtype, scale=1.0, chunk=64) -> gdn_dims:
    return gdn_dims(int(B), int(T), int(Hk), int(Hv), int(Dk), int(Dv), int(chunk),
                    _dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype), float(scale))


def gdn_chunk_fwd_workspace_bytes(dims: gdn_dims) -> int:
    return int(lib().gdn_chunk_fwd_workspace_bytes(ctypes.byref(dims)))


def alloc_workspace(dims: gdn_dims, device="cuda") -> torch.Tensor:
    """A device buffer of the required workspace size (torch's allocator aligns to 512 B)."""
    n = gdn_chunk_fwd_workspace_bytes(dims)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def gdn2_chunk_fwd_workspace_bytes(dims: gdn_dims) -> int:
    return int(lib().gdn2_chunk_fwd_workspace_bytes(ctypes.byref(dims)))


def alloc_workspace_gdn2(dims: gdn_dims, device="cuda") -> torch.Tensor:
    """A device buffer of the workspace size gdn2_chunk_fwd needs."""
    n = gdn2_chunk_fwd_workspace_bytes(dims)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def gdn_chunk_fwd(q, k, v, a, b, A_log, dt_bias, initial_state=None, *, scale: float = 1.0,
                  out=None, final_state=None, output_final_state: bool = True, workspace=None,
                  stream=None, stage_events: Optional[Sequence[int]] = None
                  ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked prefill.  q, k [B,T,Hk,Dk]; v [B,T,Hv,Dv]; a, b [B,T,Hv] fp32;
    A_log, dt_bias [Hv] fp32; initial_state [B,Hv,Dk,Dv] fp32 or None.
    Returns (out [B,T,Hv,Dv], final_state [B,Hv,Dk,Dv] or None)."""
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    dims = make_dims(B, T, Hk, Hv, Dk, Dv, q.dtype, scale)
    f32, dt = torch.float32, q.dtype
    _validate(q.device, [
        ("q", q, None, None), ("k", k, q.shape, dt), ("v", v, (B, T, Hv, Dv), dt),
        ("a", a, (B, T, Hv), f32), ("b", b, (B, T, Hv), f32), ("A_log", A_log, (Hv,), f32),
        ("dt_bias", dt_bias, (Hv,), f32), ("initial_state", initial_state, (B, Hv, Dk, Dv), f32),
        ("out", out, (B, T, Hv, Dv), dt), ("final_state", final_state, (B, Hv, Dk, Dv), f32),
        _workspace_spec(workspace, gdn_chunk_fwd_workspace_bytes(dims))])
    if out is None:
        out = torch.empty((B, T, Hv, Dv), dtype=q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, Hv, Dk, Dv), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(dims, q.device)
    ev = None
    if stage_events is not None:
        ev = (ctypes.c_void_p * (GDN_CHUNK_FWD_STAGES + 1))(*stage_events)
    st = lib().gdn_chunk_fwd_timed(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
        _ptr(initial_state), _ptr(out), _ptr(final_state), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream), ev)
    _check(st)
    return out, final_state


NOALLOC_MAX_WORKSPACE_BYTES = 128 << 20  # GDN_NOALLOC_MAX_WORKSPACE_BYTES


def gdn_chunk_fwd_noalloc(q, k, v, a, b, A_log, dt_bias, initial_state=None, *, scale: float = 1.0,
                          out=None, final_state=None, output_final_state: bool = True, stream=None
                          ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """gdn_chunk_fwd without a workspace: the library's own device scratch is used (see
    gdn_chunk_fwd_noalloc in include/gdn.h: bounded size, one per GPU, shared by all calls
    on that GPU).  Pass out (and final_state) to allocate nothing at all."""
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    dims = make_dims(B, T, Hk, Hv, Dk, Dv, q.dtype, scale)
    f32, dt = torch.float32, q.dtype
    _validate(q.device, [
        ("q", q, None, None), ("k", k, q.shape, dt), ("v", v, (B, T, Hv, Dv), dt),
        ("a", a, (B, T, Hv), f32), ("b", b, (B, T, Hv), f32), ("A_log", A_log, (Hv,), f32),
        ("dt_bias", dt_bias, (Hv,), f32), ("initial_state", initial_state, (B, Hv, Dk, Dv), f32),
        ("out", out, (B, T, Hv, Dv), dt), ("final_state", final_state, (B, Hv, Dk, Dv), f32)])
    if out is None:
        out = torch.empty((B, T, Hv, Dv), dtype=q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, Hv, Dk, Dv), dtype=torch.float32, device=q.device)
    st = lib().gdn_chunk_fwd_noalloc(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
        _ptr(initial_state), _ptr(out), _ptr(final_state), _stream(stream))
    _check(st)
    return out, final_state


def gdn2_chunk_fwd(q, k, v, a, A_log, erase, write, initial_state=None, *, scale: float = 1.0,
                   out=None, final_state=None, output_final_state: bool = True, workspace=None,
                   stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Gated DeltaNet-2 chunked prefill, bfloat16 or float32 (q's dtype).  q, k [B,T,Hk,Dk];
    v [B,T,Hv,Dv]; a, erase [B,T,Hv,Dk]; write [B,T,Hv,Dv] (all in q's dtype); A_log
    [Hv,Dk] fp32; initial_state [B,Hv,Dk,Dv] fp32 or None.  Returns (out [B,T,Hv,Dv] in
    q's dtype, final_state or None)."""
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    dims = make_dims(B, T, Hk, Hv, Dk, Dv, q.dtype, scale)
    f32, dt = torch.float32, q.dtype
    _validate(q.device, [
        ("q", q, None, None), ("k", k, q.shape, dt), ("v", v, (B, T, Hv, Dv), dt),
        ("a", a, (B, T, Hv, Dk), dt), ("erase", erase, (B, T, Hv, Dk), dt),
        ("write", write, (B, T, Hv, Dv), dt), ("A_log", A_log, (Hv, Dk), f32),
        ("initial_state", initial_state, (B, Hv, Dk, Dv), f32), ("out", out, (B, T, Hv, Dv), dt),
        ("final_state", final_state, (B, Hv, Dk, Dv), f32),
        _workspace_spec(workspace, gdn2_chunk_fwd_workspace_bytes(dims))])
    if out is None:
        out = torch.empty((B, T, Hv, Dv), dtype=q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, Hv, Dk, Dv), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace_gdn2(dims, device=q.device)
    st = lib().gdn2_chunk_fwd(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(A_log), _ptr(erase), _ptr(write),
        _ptr(initial_state), _ptr(out), _ptr(final_state), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st)
    return out, final_state


def gdn2_chunk_bwd_workspace_bytes(dims: gdn_dims) -> int:
    return int(lib().gdn2_chunk_bwd_workspace_bytes(ctypes.byref(dims)))


def gdn2_chunk_bwd(q, k, v, a, A_log, erase, write, initial_state, d_out, d_final_state=None, *,
                   scale: float = 1.0, output_d_initial_state: bool = True, workspace=None,
                   stream=None, grads=None, stage_events=None) -> dict:
    """Gradient of gdn2_chunk_fwd: the vector-Jacobian products of (out, final_state) with
    (d_out [B,T,Hv,Dv] bfloat16, d_final_state [B,Hv,Dk,Dv] fp32 or None).  Same inputs as
    gdn2_chunk_fwd.  Returns a dict of float32 tensors: dq, dk [B,T,Hk,Dk]; dv, d_write
    [B,T,Hv,Dv]; da, d_erase [B,T,Hv,Dk]; dA_log [Hv,Dk]; d_initial_state [B,Hv,Dk,Dv]
    (or None when output_d_initial_state is False).  grads: an earlier result to write
    into instead; stage_events: a StageEvents(GDN2_CHUNK_BWD_STAGES) to time each launch."""
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    dims = make_dims(B, T, Hk, Hv, Dk, Dv, q.dtype, scale)
    f32, dt = torch.float32, q.dtype
    gshapes = {"dq": (B, T, Hk, Dk), "dk": (B, T, Hk, Dk), "dv": (B, T, Hv, Dv), "da": (B, T, Hv, Dk),
               "d_erase": (B, T, Hv, Dk), "d_write": (B, T, Hv, Dv), "dA_log": (Hv, Dk),
               "d_initial_state": (B, Hv, Dk, Dv)}
    if grads is not None:
        if not isinstance(grads, dict):
            raise TypeError("grads must be a dict of tensors")
        missing = [n for n in gshapes if n not in grads or (grads[n] is None and n != "d_initial_state")]
        if missing:
            raise ValueError(f"grads is missing {missing}")
    _validate(q.device, [
        ("q", q, None, None), ("k", k, q.shape, dt), ("v", v, (B, T, Hv, Dv), dt),
        ("a", a, (B, T, Hv, Dk), dt), ("erase", erase, (B, T, Hv, Dk), dt),
        ("write", write, (B, T, Hv, Dv), dt), ("A_log", A_log, (Hv, Dk), f32),
        ("initial_state", initial_state, (B, Hv, Dk, Dv), f32), ("d_out", d_out, (B, T, Hv, Dv), dt),
        ("d_final_state", d_final_state, (B, Hv, Dk, Dv), f32),
        *([(f"grads['{n}']", grads[n], shp, f32) for n, shp in gshapes.items()] if grads is not None else []),
        _workspace_spec(workspace, gdn2_chunk_bwd_workspace_bytes(dims))])
    dev = q.device
    g = grads if grads is not None else {n: torch.empty(shp, dtype=f32, device=dev)
                                         for n, shp in gshapes.items()
                                         if n != "d_initial_state" or output_d_initial_state}
    g.setdefault("d_initial_state", None)
    if workspace is None:
        workspace = torch.empty(max(gdn2_chunk_bwd_workspace_bytes(dims), 1), dtype=torch.uint8, device=dev)
    st = lib().gdn2_chunk_bwd_timed(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(A_log), _ptr(erase), _ptr(write),
        _ptr(initial_state), _ptr(d_out), _ptr(d_final_state), _ptr(g["dq"]), _ptr(g["dk"]),
        _ptr(g["dv"]), _ptr(g["da"]), _ptr(g["d_erase"]), _ptr(g["d_write"]), _ptr(g["dA_log"]),
        _ptr(g["d_initial_state"]), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream), None if stage_events is None else stage_events._arr)
    _check(st)
    return g


def gdn_recurrent_step(q, k, v, a, b, A_log, dt_bias, state, *, scale: float = 1.0, out=None,
                       stream=None) -> torch.Tensor:
    """One decode step, state updated in place.  q, k [B,Hk,Dk]; v [B,Hv,Dv];
    a, b [B,Hv] fp32; state [B,Hv,Dk,Dv] fp32.  Returns out [B,Hv,Dv]."""
    B, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    dims = make_dims(B, 1, Hk, Hv, Dk, Dv, q.dtype, scale)
    f32, dt = torch.float32, q.dtype
    _validate(q.device, [
        ("q", q, None, None), ("k", k, q.shape, dt), ("v", v, (B, Hv, Dv), dt), ("a", a, (B, Hv), f32),
        ("b", b, (B, Hv), f32), ("A_log", A_log, (Hv,), f32), ("dt_bias", dt_bias, (Hv,), f32),
        ("state", state, (B, Hv, Dk, Dv), f32), ("out", out, (B, Hv, Dv), dt)])
    if state is None:
        raise ValueError("state is required")
    if out is None:
        out = torch.empty((B, Hv, Dv), dtype=q.dtype, device=q.device)
    st = lib().gdn_recurrent_step(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                  _ptr(A_log), _ptr(dt_bias), _ptr(state), _ptr(out), _stream(stream))
    _check(st)
    return out


def gdn2_recurrent_step(q, k, v, a, A_log, erase, write, state, *, scale: float = 1.0, out=None,
                        stream=None) -> torch.Tensor:
    """One Gated DeltaNet-2 decode step, state updated in place.  q, k [B,Hk,Dk];
    v [B,Hv,Dv]; a, erase [B,Hv,Dk] and write [B,Hv,Dv] in the dtype of q; A_log
    [Hv,Dk] fp32; state [B,Hv,Dk,Dv] fp32.  Returns out [B,Hv,Dv]."""
    B, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    dims = make_dims(B, 1, Hk, Hv, Dk, Dv, q.dtype, scale)
    f32, dt = torch.float32, q.dtype
    _validate(q.device, [
        ("q", q, None, None), ("k", k, q.shape, dt), ("v", v, (B, Hv, Dv), dt), ("a", a, (B, Hv, Dk), dt),
        ("erase", erase, (B, Hv, Dk), dt), ("write", write, (B, Hv, Dv), dt), ("A_log", A_log, (Hv, Dk), f32),
        ("state", state, (B, Hv, Dk, Dv), f32), ("out", out, (B, Hv, Dv), dt)])
    if state is None:
        raise ValueError("state is required")
    if out is None:
        out = torch.empty((B, Hv, Dv), dtype=q.dtype, device=q.device)
    st = lib().gdn2_recurrent_step(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(A_log),
                                   _ptr(erase), _ptr(write), _ptr(state), _ptr(out), _stream(stream))
    _check(st)
    return out


GDN_GATE_SILU, GDN_GATE_SIGMOID = 0, 1


def gdn_gated_rmsnorm(x, z, weight, *, eps: float = 1e-6, gate: str = "silu", out=None,
                      stream=None) -> torch.Tensor:
    """Gated RMS normalisation over the last axis (d = 64 or 128): x / rms(x) * weight *
    act(z), act = SiLU ("silu") or sigmoid ("sigmoid").  x and z of one shape and dtype
    (bf16 or fp32); weight [d] fp32.  out may be x (in place)."""
    d = x.shape[-1]
    gates = {"silu": GDN_GATE_SILU, "sigmoid": GDN_GATE_SIGMOID}
    if gate not in gates:
        raise ValueError(f"gate must be one of {sorted(gates)}")
    _validate(x.device, [("x", x, None, None), ("z", z, x.shape, x.dtype),
                         ("weight", weight, (d,), torch.float32), ("out", out, x.shape, x.dtype)])
    if out is None:
        out = torch.empty_like(x)
    rows = x.numel() // d if d else 0
    dt = GDN_F32 if x.dtype == torch.float32 else GDN_BF16 if x.dtype == torch.bfloat16 else -1
    st = lib().gdn_gated_rmsnorm(rows, d, dt, _ptr(x), _ptr(z), _ptr(weight), float(eps), gates[gate],
                                 _ptr(out), _stream(stream))
    _check(st)
    return out


GDN_ACT_NONE, GDN_ACT_SILU = 0, 1


def gdn_causal_conv1d(x, weight, bias=None, conv_state=None, *, Hk: int, Hv: int, Dk: int, Dv: int,
                      activation: str = "silu", conv_state_out=None, output_conv_state: bool = True,
                      q=None, k=None, v=None, stream=None):
    """Depthwise causal conv1d (kernel 4) + SiLU over the mixed projection x [B,T,C]
    (C = 2 Hk Dk + Hv Dv, channels q | k | v), split into q, k [B,T,Hk,Dk] and v [B,T,Hv,Dv].
    weight [C,4] fp32, bias [C] fp32 or None, conv_state [B,3,C] (x dtype) or None.
    Returns (q, k, v, conv_state_out or None); conv_state_out may be conv_state."""
    B, T, C = x.shape
    K = weight.shape[1] if weight.dim() == 2 else 0
    if C != 2 * Hk * Dk + Hv * Dv:
        raise ValueError("x's last axis must be 2 Hk Dk + Hv Dv")
    acts = {"silu": GDN_ACT_SILU, "none": GDN_ACT_NONE}
    if activation not in acts:
        raise ValueError(f"activation must be one of {sorted(acts)}")
    f32, dt = torch.float32, x.dtype
    _validate(x.device, [
        ("x", x, None, None), ("weight", weight, (C, K), f32), ("bias", bias, (C,), f32),
        ("conv_state", conv_state, (B, K - 1, C), dt), ("conv_state_out", conv_state_out, (B, K - 1, C), dt),
        ("q", q, (B, T, Hk, Dk), dt), ("k", k, (B, T, Hk, Dk), dt), ("v", v, (B, T, Hv, Dv), dt)])
    dims = make_dims(B, T, Hk, Hv, Dk, Dv, x.dtype)
    mk = lambda H, D: torch.empty((B, T, H, D), dtype=x.dtype, device=x.device)
    q = mk(Hk, Dk) if q is None else q
    k = mk(Hk, Dk) if k is None else k
    v = mk(Hv, Dv) if v is None else v
    if conv_state_out is None and output_conv_state:
        conv_state_out = torch.empty((B, K - 1, C), dtype=x.dtype, device=x.device)
    st = lib().gdn_causal_conv1d(ctypes.byref(dims), K, _ptr(x), _ptr(weight), _ptr(bias), _ptr(conv_state),
                                 _ptr(conv_state_out), acts[activation], _ptr(q), _ptr(k), _ptr(v),
                                 _stream(stream))
    _check(st)
    return q, k, v, conv_state_out


class StageEvents:
    """stages + 1 HIP events (default GDN_CHUNK_FWD_STAGES) for the timed entry points."""

    def __init__(self, stages: int = None):
        self.n = (GDN_CHUNK_FWD_STAGES if stages is None else int(stages)) + 1
        self._arr = (ctypes.c_void_p * self.n)()
        _check(lib().gdn_events_create(self.n, self._arr))

    @property
    def handles(self):
        return [self._arr[i] for i in range(self.n)]

    def stage_ms(self):
        """Elapsed ms of each stage of the last recorded call (stream must be synchronised)."""
        res = []
        for i in range(self.n - 1):
            ms = ctypes.c_float()
            _check(lib().gdn_event_elapsed_ms(self._arr[i], self._arr[i + 1], ctypes.byref(ms)))
            res.append(ms.value)
        return res

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = ctypes.c_float()
        _check(lib().gdn_event_elapsed_ms(self._arr[i], self._arr[j], ctypes.byref(ms)))
        return ms.value

    def close(self):
        if self._arr is not None:
            lib().gdn_events_destroy(self.n, self._arr)
            self._arr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
