"""Float64 CPU oracle of the Gated DeltaNet core -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the GPU library
(``gated_deltanet_sequence_amd``) and never imports it.

The arithmetic lives in ``gdn_oracle.c`` (plain token-by-token float64 loops,
built with gcc, no fast-math, ``-ffp-contract=off``); this module only widens
inputs to float64 and calls it.  ``wy_chunk.py`` holds the pages' chunkwise
(WY) form in NumPy float64, used as an independent cross-check of the token
loop.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

GCC_CMD = ["gcc", "-O3", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
           "-std=c11", "-Wall", "-Wextra", _SRC, "-o", _LIB, "-lm"]


def build() -> str:
    """Compile the C oracle with gcc into ``oracle/liboracle.so``."""
    subprocess.run(GCC_CMD, check=True)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    D = ctypes.POINTER(ctypes.c_double)
    i = ctypes.c_int
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_softplus.restype = ctypes.c_double
    lib.oracle_softplus.argtypes = [ctypes.c_double]
    lib.oracle_sigmoid.restype = ctypes.c_double
    lib.oracle_sigmoid.argtypes = [ctypes.c_double]
    lib.oracle_gdn_gates.argtypes = [ctypes.c_long, i, D, D, D, D, D, D]
    lib.oracle_gdn_core.argtypes = [i] * 6 + [D] * 5 + [ctypes.c_double, D, D, D]
    lib.oracle_gdn_fwd.argtypes = [i] * 6 + [D] * 7 + [ctypes.c_double, D, D, D]
    lib.oracle_gdn2_gates.argtypes = [ctypes.c_long, i, i, i, D, D, D, D, D, D, D]
    lib.oracle_gdn2_core.argtypes = [i] * 6 + [D] * 6 + [ctypes.c_double, D, D, D]
    lib.oracle_gdn2_fwd.argtypes = [i] * 6 + [D] * 7 + [ctypes.c_double, D, D, D]
    lib.oracle_gdn2_bwd.argtypes = [i] * 6 + [D] * 7 + [ctypes.c_double] + [D] * 11
    lib.oracle_gated_rmsnorm.argtypes = [ctypes.c_long, i, D, D, D, ctypes.c_double, i, D]
    lib.oracle_causal_conv1d.argtypes = [i, i, i, i, D, D, D, D, i, D, D]
    _lib = lib
    return lib


def f64(x) -> np.ndarray:
    """Widen a torch tensor or array (fp32/bf16/fp64) exactly to a C-contiguous float64 array."""
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(x: Optional[np.ndarray]):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def softplus(x: float) -> float:
    return float(_load().oracle_softplus(float(x)))


def sigmoid(x: float) -> float:
    return float(_load().oracle_sigmoid(float(x)))


def gdn_gates(a, b, A_log, dt_bias):
    """g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b); a, b [..., Hv]."""
    a, b, A_log, dt_bias = f64(a), f64(b), f64(A_log), f64(dt_bias)
    Hv = a.shape[-1]
    g = np.empty_like(a)
    beta = np.empty_like(a)
    _load().oracle_gdn_gates(a.size // Hv, Hv, _p(a), _p(b), _p(A_log), _p(dt_bias), _p(g), _p(beta))
    return g, beta


def gdn_core(q, k, v, g, beta, S0=None, scale: float = 1.0):
    """Token-by-token gated delta rule from explicit log decay g and beta.

    q, k [B,T,Hk,Dk]; v [B,T,Hv,Dv]; g, beta [B,T,Hv]; S0 [B,Hv,Dk,Dv] or None.
    Returns (out [B,T,Hv,Dv], S_T [B,Hv,Dk,Dv]) in float64.
    """
    q, k, v, g, beta, S0 = (f64(t) for t in (q, k, v, g, beta, S0))
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    out = np.empty((B, T, Hv, Dv))
    ST = np.empty((B, Hv, Dk, Dv))
    _load().oracle_gdn_core(B, T, Hk, Hv, Dk, Dv, _p(q), _p(k), _p(v), _p(g), _p(beta),
                            float(scale), _p(S0), _p(out), _p(ST))
    return out, ST


def gdn_fwd(q, k, v, a, b, A_log, dt_bias, S0=None, scale: float = 1.0):
    """GDN forward from raw logits (gates + recurrence).  Returns (out, S_T) float64."""
    q, k, v, a, b, A_log, dt_bias, S0 = (f64(t) for t in (q, k, v, a, b, A_log, dt_bias, S0))
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    out = np.empty((B, T, Hv, Dv))
    ST = np.empty((B, Hv, Dk, Dv))
    _load().oracle_gdn_fwd(B, T, Hk, Hv, Dk, Dv, _p(q), _p(k), _p(v), _p(a), _p(b), _p(A_log),
                           _p(dt_bias), float(scale), _p(S0), _p(out), _p(ST))
    return out, ST


def gdn_step(q, k, v, a, b, A_log, dt_bias, S, scale: float = 1.0):
    """One decode step: one token of the recurrence.

    q, k [B,Hk,Dk]; v [B,Hv,Dv]; a, b [B,Hv]; S [B,Hv,Dk,Dv].
    Returns (out [B,Hv,Dv], S_new [B,Hv,Dk,Dv]) in float64.
    """
    q, k, v, a, b = (f64(t)[:, None] for t in (q, k, v, a, b))
    out, ST = gdn_fwd(q, k, v, a, b, A_log, dt_bias, S0=S, scale=scale)
    return out[:, 0], ST


def gdn2_gates(a, A_log, erase, write):
    """Channel-wise log decay, erase gate and write gate from raw logits.

    a, erase [..., Hv, Dk]; write [..., Hv, Dv]; A_log [Hv, Dk].
    """
    a, A_log, erase, write = f64(a), f64(A_log), f64(erase), f64(write)
    Hv, Dk = a.shape[-2], a.shape[-1]
    Dv = write.shape[-1]
    g = np.empty_like(a)
    eb = np.empty_like(a)
    wb = np.empty_like(write)
    _load().oracle_gdn2_gates(a.size // (Hv * Dk), Hv, Dk, Dv, _p(a), _p(A_log), _p(erase),
                              _p(write), _p(g), _p(eb), _p(wb))
    return g, eb, wb


def gdn2_core(q, k, v, g, eb, wb, S0=None, scale: float = 1.0):
    """Token-by-token Gated Delta Rule-2 from explicit channel-wise log decay and gates."""
    q, k, v, g, eb, wb, S0 = (f64(t) for t in (q, k, v, g, eb, wb, S0))
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    out = np.empty((B, T, Hv, Dv))
    ST = np.empty((B, Hv, Dk, Dv))
    _load().oracle_gdn2_core(B, T, Hk, Hv, Dk, Dv, _p(q), _p(k), _p(v), _p(g), _p(eb), _p(wb),
                             float(scale), _p(S0), _p(out), _p(ST))
    return out, ST


def gdn2_fwd(q, k, v, a, A_log, erase, write, S0=None, scale: float = 1.0):
    """Gated DeltaNet-2 forward from raw logits.  Returns (out, S_T) float64."""
    q, k, v, a, A_log, erase, write, S0 = (f64(t) for t in (q, k, v, a, A_log, erase, write, S0))
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    out = np.empty((B, T, Hv, Dv))
    ST = np.empty((B, Hv, Dk, Dv))
    _load().oracle_gdn2_fwd(B, T, Hk, Hv, Dk, Dv, _p(q), _p(k), _p(v), _p(a), _p(A_log),
                            _p(erase), _p(write), float(scale), _p(S0), _p(out), _p(ST))
    return out, ST


def gdn2_bwd(q, k, v, a, A_log, erase, write, d_out, S0=None, d_ST=None, scale: float = 1.0):
    """Gradient of gdn2_fwd: the vector-Jacobian products of (out, S_T) with (d_out, d_ST)
    (d_ST None = 0), by reverse-mode differentiation of the token loop.  Returns a dict of
    float64 arrays: dq, dk [B,T,Hk,Dk]; dv, d_write [B,T,Hv,Dv]; da, d_erase [B,T,Hv,Dk];
    dA_log [Hv,Dk]; dS0 [B,Hv,Dk,Dv]."""
    q, k, v, a, A_log, erase, write, d_out, S0, d_ST = (
        f64(t) for t in (q, k, v, a, A_log, erase, write, d_out, S0, d_ST))
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    r = {"dq": np.empty((B, T, Hk, Dk)), "dk": np.empty((B, T, Hk, Dk)),
         "dv": np.empty((B, T, Hv, Dv)), "da": np.empty((B, T, Hv, Dk)),
         "d_erase": np.empty((B, T, Hv, Dk)), "d_write": np.empty((B, T, Hv, Dv)),
         "dA_log": np.empty((Hv, Dk)), "dS0": np.empty((B, Hv, Dk, Dv))}
    _load().oracle_gdn2_bwd(B, T, Hk, Hv, Dk, Dv, _p(q), _p(k), _p(v), _p(a), _p(A_log),
                            _p(erase), _p(write), float(scale), _p(S0), _p(d_out), _p(d_ST),
                            _p(r["dq"]), _p(r["dk"]), _p(r["dv"]), _p(r["da"]), _p(r["d_erase"]),
                            _p(r["d_write"]), _p(r["dA_log"]), _p(r["dS0"]))
    return r


GATE_SILU, GATE_SIGMOID = 0, 1


def gated_rmsnorm(x, z, weight, eps: float, gate: int = GATE_SILU):
    """Gated RMS normalisation over the last axis: x / rms(x) * weight * act(z),
    act = SiLU (GATE_SILU) or sigmoid (GATE_SIGMOID).  Returns float64."""
    x, z, weight = f64(x), f64(z), f64(weight)
    d = x.shape[-1]
    if z.shape != x.shape or weight.shape != (d,):
        raise ValueError("shape mismatch")
    y = np.empty_like(x)
    _load().oracle_gated_rmsnorm(x.size // d, d, _p(x), _p(z), _p(weight), float(eps), int(gate), _p(y))
    return y


def causal_conv1d(x, weight, bias=None, state=None, silu: bool = True):
    """Depthwise causal convolution over time (+ SiLU).  x [B,T,C]; weight [C,K]; bias [C]
    or None; state [B,K-1,C] (the inputs before token 0) or None.  Returns (y [B,T,C],
    state_out [B,K-1,C]) in float64."""
    x, weight = f64(x), f64(weight)
    bias, state = f64(bias), f64(state)
    B, T, C = x.shape
    K = weight.shape[1]
    y = np.empty((B, T, C))
    st = np.empty((B, K - 1, C))
    _load().oracle_causal_conv1d(B, T, C, K, _p(x), _p(weight), _p(bias), _p(state), int(bool(silu)),
                                 _p(y), _p(st))
    return y, st


def rel_l2(x, ref) -> float:
    """||x - ref||_2 / ||ref||_2 over the whole tensor, in float64."""
    x, ref = f64(x), f64(ref)
    den = float(np.sqrt(np.sum(ref * ref)))
    num = float(np.sqrt(np.sum((x - ref) ** 2)))
    return num / den if den > 0 else num
