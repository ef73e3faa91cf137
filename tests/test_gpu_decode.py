"""GPU parity of the recurrent decode step (gdn_recurrent_step) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import GDNSpec, WORKLOADS
from tests.gpu_util import (BF16_DECODE_BOUNDS, BF16_ROUNDED_TOL, TOL, Stats, accumulate_out, accumulate_state,
                            assert_close, check_stats, log, oracle_prefill, to_dev)

pytestmark = pytest.mark.gpu


def run_steps(spec: GDNSpec, inp, nsteps=None, scale=1.0):
    """Feed tokens 0..nsteps-1 one at a time through the decode step; returns (out, state)."""
    import gated_deltanet_sequence_amd as gdn
    d = to_dev(inp)
    nsteps = spec.T if nsteps is None else nsteps
    S = d["S0"].clone() if d["S0"] is not None else torch.zeros(
        (spec.B, spec.Hv, spec.Dk, spec.Dv), dtype=torch.float32, device="cuda")
    outs = []
    for t in range(nsteps):
        o = gdn.gdn_recurrent_step(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                                   d["v"][:, t].contiguous(), d["a"][:, t].contiguous(),
                                   d["b"][:, t].contiguous(), d["A_log"], d["dt_bias"], S, scale=scale)
        outs.append(o)
    torch.cuda.synchronize()
    return torch.stack(outs, dim=1).cpu(), S.cpu()


@pytest.mark.parametrize("dtype,Dk,Dv", [("f32", 64, 64), ("f32", 128, 128), ("f32", 64, 128),
                                         ("bf16", 128, 128), ("bf16", 128, 64)])
def test_steps_match_oracle(dtype, Dk, Dv):
    spec = GDNSpec(B=3, T=20, Hk=2, Hv=4, Dk=Dk, Dv=Dv, dtype=dtype, seed=300 + Dk + Dv,
                   init_state=True)
    log(f"[decode] {spec}")
    inp = synth.make_inputs(spec)
    out, S = run_steps(spec, inp)
    o_ref, s_ref = oracle_prefill(inp)
    assert_close("out", out, o_ref, TOL[dtype])
    assert_close("state", S, s_ref, TOL[dtype])


def test_tiny_f32_by_steps():
    """The tiny fp32 forward (T=256) token by token through the step == oracle forward."""
    spec = WORKLOADS["tiny_f32"]
    log(f"[decode tiny] {spec}")
    inp = synth.make_inputs(spec)
    out, S = run_steps(spec, inp)
    o_ref, s_ref = oracle_prefill(inp)
    assert_close("out", out, o_ref, TOL["f32"])
    assert_close("state", S, s_ref, TOL["f32"])


def test_scale_and_single_step_f32():
    spec = GDNSpec(B=5, T=1, Hk=1, Hv=3, Dk=128, Dv=64, dtype="f32", seed=310, init_state=True)
    log(f"[decode scale] {spec}")
    inp = synth.make_inputs(spec)
    out, S = run_steps(spec, inp, scale=0.125)
    o_ref, s_ref = oracle_prefill(inp, scale=0.125)
    assert_close("out", out, o_ref, TOL["f32"])
    assert_close("state", S, s_ref, TOL["f32"])


def test_decode_b256_64_steps():
    """B=256 sequences, 16/64 heads, d=128, bf16, state N(0, 0.02^2) (1 GiB), 64 consecutive
    steps in place -- the timed decode workload.  The oracle over all 16384 (sequence, value
    head) pairs, 32 sequences at a time: all 64 outputs and the state after step 64."""
    spec = WORKLOADS["decode_b256"]
    log(f"[decode] {spec}")
    inp = synth.make_inputs(spec)
    out, S = run_steps(spec, inp)
    assert torch.isfinite(S).all() and torch.isfinite(out.float()).all()
    so, ss = Stats(), Stats()
    for b0 in range(0, spec.B, 32):
        sl = synth.key_head_slice(inp, spec, b0, b0 + 32, 0, spec.Hk)
        o_ref, s_ref = oracle_prefill(sl)
        accumulate_out(so, out[b0:b0 + 32], o_ref, b0=b0, bf16=True)
        accumulate_state(ss, S[b0:b0 + 32], s_ref, b0=b0)
    check_stats("out (16384 heads x 64 steps)", so, **BF16_DECODE_BOUNDS, rounded_tol=BF16_ROUNDED_TOL)
    check_stats("state (16384 heads)", ss, TOL["bf16"], head_tol=TOL["bf16"])


@pytest.mark.parametrize("dtype,Dk,Dv", [("f32", 128, 128), ("bf16", 128, 128), ("bf16", 64, 128)])
def test_ragged_persistent_tail(dtype, Dk, Dv):
    """B*Hv = 1072 heads: more than any resident grid (at most 4 work-groups on each of
    256 CUs) and not a multiple of 256, so the persistent loop walks several heads per
    work-group and ends on a partial sweep."""
    spec = GDNSpec(B=67, T=3, Hk=4, Hv=16, Dk=Dk, Dv=Dv, dtype=dtype, seed=320 + Dk, init_state=True)
    log(f"[decode ragged] {spec}")
    inp = synth.make_inputs(spec)
    out, S = run_steps(spec, inp)
    o_ref, s_ref = oracle_prefill(inp)
    assert_close("out", out, o_ref, TOL[dtype])
    assert_close("state", S, s_ref, TOL[dtype])
