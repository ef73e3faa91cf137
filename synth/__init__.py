"""Seeded synthetic inputs for the Gated DeltaNet core.

This module draws random tensors and nothing else: it holds none of the
method's arithmetic (no gates, no decay, no recurrence).  The GPU path, the
oracle, the tests and the benchmark all consume the tensors it returns, so
both sides of every parity check see identical bytes.

Recipe (one stream per tensor, NumPy PCG64 seeded with ``[seed, tensor_id]``):

* values are drawn in float64, in row-major order of the tensor, slab by slab
  along the leading axes;
* q and k are L2-normalised per (batch, token, key head) vector in float64;
* everything is rounded to float32, then (for bf16 workloads) to bfloat16
  with round-to-nearest-even;
* gate logits a, b ~ N(0, 1); A_log ~ U(lo, hi) (default U(0, ln 16));
  dt_bias ~ U(-1, 1); the initial state, when present, is N(0, sigma^2) with
  sigma = 0.02, stored in float32.

The distributions follow the Qwen3.5 linear-attention layer shapes: 16 key
heads shared by 64 value heads of size 128 (page "Qwen3.5 ... GDN" at
10100.com, section one), with the decay parametrisation of the dingfen.github.io
page, section 9.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np
import torch

# tensor ids of the per-tensor random streams
TID_A_LOG, TID_DT_BIAS, TID_Q, TID_K, TID_V, TID_A, TID_B, TID_S0, TID_ERASE, TID_WRITE = range(10)
TID_NORM_X, TID_NORM_Z, TID_NORM_W = 10, 11, 12
TID_CONV_X, TID_CONV_W, TID_CONV_B, TID_CONV_S = 13, 14, 15, 16
TID_DOUT, TID_DST = 17, 18

_SLAB = 1 << 22  # values drawn per slab (bounds the float64 working set)


@dataclass(frozen=True)
class GDNSpec:
    """Shape and distribution of one synthetic Gated DeltaNet workload."""

    B: int
    T: int
    Hk: int
    Hv: int
    Dk: int
    Dv: int
    dtype: str = "bf16"          # "f32" or "bf16": dtype of q, k, v (and of the output)
    seed: int = 0
    init_state: bool = False     # draw S0 ~ N(0, state_sigma^2)
    state_sigma: float = 0.02
    a_log_lo: float = 0.0
    a_log_hi: float = math.log(16.0)
    variant: str = "gdn"         # "gdn" or "gdn2"
    chunk: int = 64

    def with_(self, **kw) -> "GDNSpec":
        return replace(self, **kw)

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"f32": torch.float32, "bf16": torch.bfloat16}[self.dtype]


# Named workloads (sizes as stated for each).
WORKLOADS: Dict[str, GDNSpec] = {
    # tiny fp32 forward: parity at 1e-5
    "tiny_f32": GDNSpec(B=1, T=256, Hk=2, Hv=2, Dk=64, Dv=64, dtype="f32", seed=100),
    # Qwen3.5-shaped prefill, T=4096, 16 key / 64 value heads, d=128, bf16
    "prefill_t4096": GDNSpec(B=1, T=4096, Hk=16, Hv=64, Dk=128, Dv=128, dtype="bf16", seed=101),
    # long-context prefill, two sequences of 65536 tokens, nonzero initial state
    "prefill_long": GDNSpec(B=2, T=65536, Hk=16, Hv=64, Dk=128, Dv=128, dtype="bf16", seed=102,
                            init_state=True),
    # decode: 256 sequences, 64 consecutive one-token steps (T counts the steps)
    "decode_b256": GDNSpec(B=256, T=64, Hk=16, Hv=64, Dk=128, Dv=128, dtype="bf16", seed=103,
                           init_state=True),
    # Gated DeltaNet-2 prefill, T=8192
    "gdn2_t8192": GDNSpec(B=1, T=8192, Hk=16, Hv=64, Dk=128, Dv=128, dtype="bf16", seed=104,
                          variant="gdn2"),
    # Gated DeltaNet-2 decode: 256 sequences, 16 distinct one-token steps, state N(0, 0.02^2)
    "decode_gdn2_b256": GDNSpec(B=256, T=16, Hk=16, Hv=64, Dk=128, Dv=128, dtype="bf16", seed=105,
                                init_state=True, variant="gdn2"),
}

# Stress variants: slow decay keeps the carried state alive across chunks.
SLOW_DECAY = dict(a_log_lo=math.log(2e-3), a_log_hi=math.log(3e-2))


def _rng(seed: int, tid: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(tid)])


def _normal_rows(rng: np.random.Generator, shape, l2_normalise: bool) -> np.ndarray:
    """Draw N(0,1) float64 values of ``shape`` slab by slab; return float32.

    When ``l2_normalise`` is set, each vector along the last axis is divided by
    its float64 Euclidean norm before the float32 rounding.
    """
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1, shape[-1])
    rows_per_slab = max(1, _SLAB // shape[-1])
    for r0 in range(0, flat.shape[0], rows_per_slab):
        r1 = min(flat.shape[0], r0 + rows_per_slab)
        x = rng.standard_normal((r1 - r0, shape[-1]))
        if l2_normalise:
            x /= np.sqrt(np.sum(x * x, axis=1, keepdims=True))
        flat[r0:r1] = x
    return out


def _to_torch(x32: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    t = torch.from_numpy(x32)
    return t if dtype == torch.float32 else t.to(dtype)


def make_inputs(spec: GDNSpec) -> Dict[str, Optional[torch.Tensor]]:
    """Return the CPU tensors of one workload, in the library's layouts.

    gdn:  q, k [B,T,Hk,Dk]; v [B,T,Hv,Dv] (spec dtype); a, b [B,T,Hv] fp32;
          A_log, dt_bias [Hv] fp32; S0 [B,Hv,Dk,Dv] fp32 or None.
    gdn2: q, k, v as above; a, erase [B,T,Hv,Dk] and write [B,T,Hv,Dv] (spec
          dtype); A_log [Hv,Dk] fp32; S0 as above.
    """
    s = spec
    dt = s.torch_dtype
    out: Dict[str, Optional[torch.Tensor]] = {}
    out["q"] = _to_torch(_normal_rows(_rng(s.seed, TID_Q), (s.B, s.T, s.Hk, s.Dk), True), dt)
    out["k"] = _to_torch(_normal_rows(_rng(s.seed, TID_K), (s.B, s.T, s.Hk, s.Dk), True), dt)
    out["v"] = _to_torch(_normal_rows(_rng(s.seed, TID_V), (s.B, s.T, s.Hv, s.Dv), False), dt)
    if s.variant == "gdn":
        out["a"] = _to_torch(_normal_rows(_rng(s.seed, TID_A), (s.B, s.T, s.Hv), False), torch.float32)
        out["b"] = _to_torch(_normal_rows(_rng(s.seed, TID_B), (s.B, s.T, s.Hv), False), torch.float32)
        out["A_log"] = torch.from_numpy(
            _rng(s.seed, TID_A_LOG).uniform(s.a_log_lo, s.a_log_hi, size=(s.Hv,)).astype(np.float32))
        out["dt_bias"] = torch.from_numpy(
            _rng(s.seed, TID_DT_BIAS).uniform(-1.0, 1.0, size=(s.Hv,)).astype(np.float32))
    elif s.variant == "gdn2":
        out["a"] = _to_torch(_normal_rows(_rng(s.seed, TID_A), (s.B, s.T, s.Hv, s.Dk), False), dt)
        out["erase"] = _to_torch(_normal_rows(_rng(s.seed, TID_ERASE), (s.B, s.T, s.Hv, s.Dk), False), dt)
        out["write"] = _to_torch(_normal_rows(_rng(s.seed, TID_WRITE), (s.B, s.T, s.Hv, s.Dv), False), dt)
        out["A_log"] = torch.from_numpy(
            _rng(s.seed, TID_A_LOG).uniform(s.a_log_lo, s.a_log_hi, size=(s.Hv, s.Dk)).astype(np.float32))
    else:
        raise ValueError(f"unknown variant {s.variant!r}")
    if s.init_state:
        x = _normal_rows(_rng(s.seed, TID_S0), (s.B, s.Hv, s.Dk, s.Dv), False)
        x *= np.float32(s.state_sigma)
        out["S0"] = torch.from_numpy(x)
    else:
        out["S0"] = None
    return out


def make_grad_inputs(spec: GDNSpec, d_state: bool = True, d_state_sigma: float = 1.0):
    """Seeded gradients of the forward's outputs: d_out [B,T,Hv,Dv] N(0,1) in the input
    dtype and d_ST [B,Hv,Dk,Dv] float32 N(0, d_state_sigma) (None when d_state is False)."""
    s = spec
    dt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    d_out = _to_torch(_normal_rows(_rng(s.seed, TID_DOUT), (s.B, s.T, s.Hv, s.Dv), False), dt)
    d_ST = None
    if d_state:
        x = _normal_rows(_rng(s.seed, TID_DST), (s.B, s.Hv, s.Dk, s.Dv), False)
        x *= np.float32(d_state_sigma)
        d_ST = torch.from_numpy(x)
    return {"d_out": d_out, "d_ST": d_ST}


def head_slice(inp: Dict[str, Optional[torch.Tensor]], spec: GDNSpec, b: int, hv: int):
    """Inputs of one (sequence, value head) pair as a B=1, Hk=Hv=1 problem.

    Pure indexing: value head ``hv`` reads key head ``hv // (Hv // Hk)``.
    """
    hk = hv // (spec.Hv // spec.Hk)
    o = {
        "q": inp["q"][b:b + 1, :, hk:hk + 1],
        "k": inp["k"][b:b + 1, :, hk:hk + 1],
        "v": inp["v"][b:b + 1, :, hv:hv + 1],
    }
    if spec.variant == "gdn":
        o["a"] = inp["a"][b:b + 1, :, hv:hv + 1]
        o["b"] = inp["b"][b:b + 1, :, hv:hv + 1]
        o["A_log"] = inp["A_log"][hv:hv + 1]
        o["dt_bias"] = inp["dt_bias"][hv:hv + 1]
    else:
        o["a"] = inp["a"][b:b + 1, :, hv:hv + 1]
        o["erase"] = inp["erase"][b:b + 1, :, hv:hv + 1]
        o["write"] = inp["write"][b:b + 1, :, hv:hv + 1]
        o["A_log"] = inp["A_log"][hv:hv + 1]
    o["S0"] = None if inp["S0"] is None else inp["S0"][b:b + 1, hv:hv + 1]
    return o


def key_head_slice(inp: Dict[str, Optional[torch.Tensor]], spec: GDNSpec, b0: int, b1: int,
                   hk0: int, hk1: int):
    """Inputs of sequences b0..b1-1 and key heads hk0..hk1-1 together with the value heads
    that read them (value heads hk0*G .. hk1*G-1, G = Hv // Hk), as a smaller problem.

    Pure indexing, like head_slice."""
    G = spec.Hv // spec.Hk
    v0, v1 = hk0 * G, hk1 * G
    o = {
        "q": inp["q"][b0:b1, :, hk0:hk1],
        "k": inp["k"][b0:b1, :, hk0:hk1],
        "v": inp["v"][b0:b1, :, v0:v1],
        "a": inp["a"][b0:b1, :, v0:v1],
        "A_log": inp["A_log"][v0:v1],
    }
    if spec.variant == "gdn":
        o["b"] = inp["b"][b0:b1, :, v0:v1]
        o["dt_bias"] = inp["dt_bias"][v0:v1]
    else:
        o["erase"] = inp["erase"][b0:b1, :, v0:v1]
        o["write"] = inp["write"][b0:b1, :, v0:v1]
    o["S0"] = None if inp["S0"] is None else inp["S0"][b0:b1, v0:v1]
    return o


def make_norm_inputs(shape, dtype: str, seed: int, x_sigma: float = 1.0):
    """Inputs of the gated RMS normalisation: x ~ N(0, x_sigma^2) and the gate z ~ N(0, 1)
    of ``shape`` (last axis = d) in ``dtype`` ("f32" or "bf16"), weight [d] ~ U(0.5, 1.5)
    float32."""
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    x = _normal_rows(_rng(seed, TID_NORM_X), tuple(shape), False)
    x *= np.float32(x_sigma)
    z = _normal_rows(_rng(seed, TID_NORM_Z), tuple(shape), False)
    w = _rng(seed, TID_NORM_W).uniform(0.5, 1.5, size=(shape[-1],)).astype(np.float32)
    return _to_torch(x, dt), _to_torch(z, dt), torch.from_numpy(w)


def make_conv_inputs(B: int, T: int, C: int, dtype: str, seed: int, K: int = 4, bias: bool = True,
                     state: bool = True):
    """Inputs of the causal conv1d prologue: the mixed projection x [B,T,C] ~ N(0,1) and the
    cached inputs state [B,K-1,C] ~ N(0,1) in ``dtype``; weight [C,K] and bias [C] ~
    U(-1/sqrt(K), 1/sqrt(K)) float32 (the usual fan-in bound of a depthwise kernel)."""
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    lim = 1.0 / math.sqrt(K)
    x = _to_torch(_normal_rows(_rng(seed, TID_CONV_X), (B, T, C), False), dt)
    w = torch.from_numpy(_rng(seed, TID_CONV_W).uniform(-lim, lim, size=(C, K)).astype(np.float32))
    b = torch.from_numpy(_rng(seed, TID_CONV_B).uniform(-lim, lim, size=(C,)).astype(np.float32)) if bias else None
    s = _to_torch(_normal_rows(_rng(seed, TID_CONV_S), (B, K - 1, C), False), dt) if state else None
    return x, w, b, s
