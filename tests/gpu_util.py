"""Helpers for the GPU parity tests: run the HIP path through the C ABI, run the
float64 oracle on the same seeded inputs, compare with relative L2 error."""
from __future__ import annotations

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
