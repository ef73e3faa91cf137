"""Helpers for the GPU parity tests: run the HIP path through the C ABI, run the
float64 oracle on the same seeded inputs, compare with relative L2 error."""
from __future__ import annotations

import math
import sys
from typing import Dict, Iterable, Optional, Tuple

import numpy as np
import torch

import oracle
import synth

TOL = {"f32": 1e-5, "bf16": 2e-3}


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(inp: Dict[str, Optional[torch.Tensor]], device="cuda"):
    return {k: (None if v is None else v.to(device).contiguous()) for k, v in inp.items()}


def gpu_prefill(spec: synth.GDNSpec, inp, scale: float = 1.0, **kw):
    import gated_deltanet_sequence_amd as gdn
    d = to_dev(inp)
    out, ST = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                                d["S0"], scale=scale, **kw)
    torch.cuda.synchronize()
    return out.cpu(), ST.cpu()


def oracle_prefill(inp, scale: float = 1.0):
    return oracle.gdn_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"],
                          inp["dt_bias"], S0=inp["S0"], scale=scale)


def oracle_heads(spec: synth.GDNSpec, inp, heads: Iterable[Tuple[int, int]], scale: float = 1.0):
    """Oracle outputs and final states of selected (sequence, value head) pairs."""
    res = {}
    for (b, hv) in heads:
        s = synth.head_slice(inp, spec, b, hv)
        o, st = oracle.gdn_fwd(s["q"], s["k"], s["v"], s["a"], s["b"], s["A_log"], s["dt_bias"],
                               S0=s["S0"], scale=scale)
        res[(b, hv)] = (o[0, :, 0], st[0, 0])
    return res


def rel(x, ref) -> float:
    return oracle.rel_l2(x, ref)


def assert_close(name: str, x, ref, tol: float):
    e = rel(x, ref)
    log(f"  {name}: rel-L2 = {e:.3e} (tol {tol:.0e})")
    assert np.isfinite(e) and e <= tol, f"{name}: rel-L2 {e:.3e} > {tol:.0e}"
    return e


def sample_heads(spec: synth.GDNSpec, n: int, seed: int = 0):
    """n distinct (b, hv) pairs, always including the first and the last."""
    rng = np.random.default_rng(seed)
    allp = [(b, h) for b in range(spec.B) for h in range(spec.Hv)]
    if n >= len(allp):
        return allp
    pick = {allp[0], allp[-1]}
    while len(pick) < n:
        pick.add(allp[int(rng.integers(len(allp)))])
    return sorted(pick)


# ---------------------------------------------------------------------------
# Full-tensor parity with per-head and per-chunk maxima.
#
# The whole-tensor relative L2 error (the stated criterion) dilutes an error
# confined to one head or one chunk, so every full comparison also reports,
# and gates, the worst (sequence, value head) and the worst (sequence, value
# head, 64-token chunk).  For bfloat16 outputs it also compares against the
# oracle rounded to bfloat16, which separates the kernel's own error from the
# rounding floor of the output type (about 1.65e-3 for these workloads).

def _t64(x) -> torch.Tensor:
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))


class Stats:
    """Sums of squares of the error and of the reference, accumulated over slices."""

    def __init__(self):
        self.num = 0.0
        self.den = 0.0
        self.worst_head = (0.0, None)
        self.worst_chunk = (0.0, None)
        self.num_r = 0.0  # against the reference rounded to bf16

    def whole(self) -> float:
        return math.sqrt(self.num / self.den) if self.den > 0 else math.sqrt(self.num)

    def rounded(self) -> float:
        return math.sqrt(self.num_r / self.den) if self.den > 0 else math.sqrt(self.num_r)


def _ratio(num: torch.Tensor, den: torch.Tensor) -> torch.Tensor:
    return torch.sqrt(num / torch.clamp(den, min=1e-300))


def accumulate_out(st: Stats, gpu, ref, b0: int = 0, h0: int = 0, chunk: int = 64, bf16: bool = False):
    """Add outputs gpu, ref [B, T, H, D] of sequences b0.. and value heads h0.. to st."""
    x, r = _t64(gpu), _t64(ref)
    assert x.shape == r.shape, (x.shape, r.shape)
    B, T, H, D = r.shape
    d2 = (x - r) ** 2
    r2 = r ** 2
    st.num += float(d2.sum())
    st.den += float(r2.sum())
    if bf16:
        rr = r.to(torch.float32).to(torch.bfloat16).to(torch.float64)
        st.num_r += float(((x - rr) ** 2).sum())
    ph = _ratio(d2.sum(dim=(1, 3)), r2.sum(dim=(1, 3)))          # [B, H]
    i = int(torch.argmax(ph))
    if float(ph.flatten()[i]) >= st.worst_head[0]:
        st.worst_head = (float(ph.flatten()[i]), (b0 + i // H, h0 + i % H))
    nc = (T + chunk - 1) // chunk
    pad = nc * chunk - T
    if pad:
        d2 = torch.nn.functional.pad(d2, (0, 0, 0, 0, 0, pad))
        r2 = torch.nn.functional.pad(r2, (0, 0, 0, 0, 0, pad))
    pc = _ratio(d2.view(B, nc, chunk, H, D).sum(dim=(2, 4)), r2.view(B, nc, chunk, H, D).sum(dim=(2, 4)))
    i = int(torch.argmax(pc))
    if float(pc.flatten()[i]) >= st.worst_chunk[0]:
        b, rest = divmod(i, nc * H)
        n, h = divmod(rest, H)
        st.worst_chunk = (float(pc.flatten()[i]), (b0 + b, h0 + h, n))


def accumulate_state(st: Stats, gpu, ref, b0: int = 0, h0: int = 0):
    """Add final states gpu, ref [B, H, Dk, Dv] of sequences b0.. and value heads h0.. to st."""
    x, r = _t64(gpu), _t64(ref)
    assert x.shape == r.shape, (x.shape, r.shape)
    B, H = r.shape[:2]
    d2 = (x - r) ** 2
    r2 = r ** 2
    st.num += float(d2.sum())
    st.den += float(r2.sum())
    ph = _ratio(d2.sum(dim=(2, 3)), r2.sum(dim=(2, 3)))
    i = int(torch.argmax(ph))
    if float(ph.flatten()[i]) >= st.worst_head[0]:
        st.worst_head = (float(ph.flatten()[i]), (b0 + i // H, h0 + i % H))


def check_stats(name: str, st: Stats, tol: float, head_tol: Optional[float] = None,
                chunk_tol: Optional[float] = None, rounded_tol: Optional[float] = None):
    """Log the whole-tensor error and the maxima; assert each against its bound."""
    e = st.whole()
    msg = f"  {name}: rel-L2 = {e:.3e} (tol {tol:.0e}); worst (b, hv) {st.worst_head[1]}: {st.worst_head[0]:.3e}"
    if st.worst_chunk[1] is not None:
        msg += f"; worst (b, hv, chunk) {st.worst_chunk[1]}: {st.worst_chunk[0]:.3e}"
    if rounded_tol is not None:
        msg += f"; vs oracle rounded to bf16: {st.rounded():.3e}"
    log(msg)
    assert math.isfinite(e) and e <= tol, f"{name}: rel-L2 {e:.3e} > {tol:.0e}"
    if head_tol is not None:
        assert st.worst_head[0] <= head_tol, f"{name}: worst head {st.worst_head}"
    if chunk_tol is not None:
        assert st.worst_chunk[0] <= chunk_tol, f"{name}: worst chunk {st.worst_chunk}"
    if rounded_tol is not None:
        assert st.rounded() <= rounded_tol, f"{name}: vs rounded oracle {st.rounded():.3e}"
    return e


# Bounds of the full bf16 comparisons: the whole tensor at the stated 2e-3; every
# (sequence, value head) at the same 2e-3; every 64-token chunk of one head at
# 4e-3 (its 8192 outputs carry the same rounding floor with a larger spread);
# and the kernel's own error, against the oracle rounded to bf16, at 1.2e-3.
BF16_BOUNDS = dict(tol=2e-3, head_tol=2e-3, chunk_tol=4e-3)
BF16_ROUNDED_TOL = 1.2e-3
# The decode workloads give each head only 16 or 64 tokens (2048 or 8192 outputs): the bf16
# rounding of the output alone spreads more per head (measured up to 1.96e-3 while the
# step's own error against the rounded oracle is 1.8e-5), so their heads are gated at 2.5e-3.
BF16_DECODE_BOUNDS = dict(tol=2e-3, head_tol=2.5e-3, chunk_tol=4e-3)
