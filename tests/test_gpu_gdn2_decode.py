"""GPU parity of the Gated DeltaNet-2 decode step (gdn2_recurrent_step) against the
float64 oracle: T steps of the kernel, each updating the state in place, against the
oracle's token loop over the same T tokens (oracle.gdn2_fwd).  Relative L2 over the
whole output and the whole final state: 1e-5 for float32 inputs, 2e-3 for bfloat16."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import GDNSpec, SLOW_DECAY, WORKLOADS
from tests.gpu_util import (BF16_DECODE_BOUNDS, BF16_ROUNDED_TOL, TOL, Stats, accumulate_out, accumulate_state,
                            assert_close, check_stats, log, to_dev)

pytestmark = pytest.mark.gpu


def run_steps(spec: GDNSpec, d, t0=0, t1=None, S=None, scale=1.0):
    """Tokens t0 .. t1-1 one at a time through the step; returns (out [B,t1-t0,Hv,Dv], S)."""
    import gated_deltanet_sequence_amd as gdn
    t1 = spec.T if t1 is None else t1
    if S is None:
        S = d["S0"].clone() if d["S0"] is not None else torch.zeros(
            (spec.B, spec.Hv, spec.Dk, spec.Dv), dtype=torch.float32, device="cuda")
    outs = []
    for t in range(t0, t1):
        sl = lambda x: x[:, t].contiguous()
        outs.append(gdn.gdn2_recurrent_step(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["a"]), d["A_log"],
                                            sl(d["erase"]), sl(d["write"]), S, scale=scale))
    torch.cuda.synchronize()
    return torch.stack(outs, dim=1), S


def oracle_gdn2(inp, scale=1.0):
    return oracle.gdn2_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["A_log"], inp["erase"],
                           inp["write"], S0=inp["S0"], scale=scale)


def check(spec: GDNSpec, scale=1.0, inp=None):
    log(f"[gdn2 decode] {spec}")
    inp = synth.make_inputs(spec) if inp is None else inp
    out, S = run_steps(spec, to_dev(inp), scale=scale)
    o_ref, s_ref = oracle_gdn2(inp, scale=scale)
    assert_close("out", out.cpu(), o_ref, TOL[spec.dtype])
    assert_close("state", S.cpu(), s_ref, TOL[spec.dtype])


def g2(**kw) -> GDNSpec:
    return GDNSpec(variant="gdn2", **kw)


@pytest.mark.parametrize("dtype,Dk,Dv", [("f32", 64, 64), ("f32", 128, 128), ("f32", 64, 128),
                                         ("bf16", 128, 128), ("bf16", 128, 64), ("bf16", 64, 128)])
def test_steps_match_oracle(dtype, Dk, Dv):
    check(g2(B=3, T=20, Hk=2, Hv=4, Dk=Dk, Dv=Dv, dtype=dtype, seed=500 + Dk + Dv, init_state=True))


def test_slow_decay_f32():
    """Per-channel decays near 1 over 40 steps: the carried state dominates."""
    check(g2(B=2, T=40, Hk=1, Hv=2, Dk=128, Dv=128, dtype="f32", seed=510, init_state=True,
             state_sigma=0.5, **SLOW_DECAY))


def test_scale_and_single_step_f32():
    check(g2(B=5, T=1, Hk=1, Hv=3, Dk=128, Dv=64, dtype="f32", seed=511, init_state=True), scale=0.125)


def test_kda_and_scalar_reductions_f32():
    """Erase = write logits, equal across channels (b = w = beta 1: the KDA rule) against the
    GDN-2 oracle; with a decay also equal across channels, against the scalar-decay oracle."""
    spec = g2(B=2, T=12, Hk=1, Hv=2, Dk=128, Dv=128, dtype="f32", seed=512, init_state=True)
    log(f"[gdn2 decode KDA] {spec}")
    inp = synth.make_inputs(spec)
    B, T, Hv, Dk, Dv = spec.B, spec.T, spec.Hv, spec.Dk, spec.Dv
    beta = inp["erase"][..., :1]
    kda = dict(inp)
    kda["erase"] = beta.expand(B, T, Hv, Dk).contiguous()
    kda["write"] = beta.expand(B, T, Hv, Dv).contiguous()
    check(spec, inp=kda)
    a_tok = inp["a"][..., :1]
    scal = dict(kda)
    scal["a"] = a_tok.expand(B, T, Hv, Dk).contiguous()
    scal["A_log"] = inp["A_log"][:, :1].expand(Hv, Dk).contiguous()
    out, S = run_steps(spec, to_dev(scal))
    o_ref, s_ref = oracle.gdn_fwd(inp["q"], inp["k"], inp["v"], a_tok[..., 0], beta[..., 0],
                                  inp["A_log"][:, 0].contiguous(), torch.zeros(Hv), S0=inp["S0"])
    assert_close("out (vs scalar-decay oracle)", out.cpu(), o_ref, TOL["f32"])
    assert_close("state (vs scalar-decay oracle)", S.cpu(), s_ref, TOL["f32"])


def test_prefill_then_steps_bf16():
    """gdn2_chunk_fwd over the first 150 tokens, then 10 steps from its final state, equal the
    oracle over all 160 tokens."""
    import gated_deltanet_sequence_amd as gdn
    spec = g2(B=2, T=160, Hk=1, Hv=2, Dk=128, Dv=128, dtype="bf16", seed=513, init_state=True)
    log(f"[gdn2 prefill + decode] {spec}")
    inp = synth.make_inputs(spec)
    d = to_dev(inp)
    T1 = 150
    sl = lambda x: x[:, :T1].contiguous()
    o1, S = gdn.gdn2_chunk_fwd(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["a"]), d["A_log"], sl(d["erase"]),
                               sl(d["write"]), d["S0"])
    o2, S = run_steps(spec, d, t0=T1, S=S)
    o_ref, s_ref = oracle_gdn2(inp)
    assert_close("out", torch.cat([o1, o2], dim=1).cpu(), o_ref, TOL["bf16"])
    assert_close("state", S.cpu(), s_ref, TOL["bf16"])


def test_state_updated_in_place():
    import gated_deltanet_sequence_amd as gdn
    spec = g2(B=1, T=1, Hk=1, Hv=2, Dk=64, Dv=64, dtype="f32", seed=514, init_state=True)
    inp = synth.make_inputs(spec)
    d = to_dev(inp)
    S = d["S0"].clone()
    ptr = S.data_ptr()
    gdn.gdn2_recurrent_step(d["q"][:, 0].contiguous(), d["k"][:, 0].contiguous(), d["v"][:, 0].contiguous(),
                            d["a"][:, 0].contiguous(), d["A_log"], d["erase"][:, 0].contiguous(),
                            d["write"][:, 0].contiguous(), S)
    torch.cuda.synchronize()
    assert S.data_ptr() == ptr and not torch.equal(S, d["S0"])


def test_decode_gdn2_b256():
    """B=256 sequences, 16/64 heads, d=128, bf16, state N(0, 0.02^2) (1 GiB), 16 consecutive
    steps in place -- the timed GDN-2 decode workload.  The oracle over all 16384 (sequence,
    value head) pairs, 32 sequences at a time: all 16 outputs and the state after the last step."""
    spec = WORKLOADS["decode_gdn2_b256"]
    log(f"[gdn2 decode] {spec}")
    inp = synth.make_inputs(spec)
    out, S = run_steps(spec, to_dev(inp))
    out, S = out.cpu(), S.cpu()
    assert torch.isfinite(S).all() and torch.isfinite(out.float()).all()
    so, ss = Stats(), Stats()
    for b0 in range(0, spec.B, 32):
        sl = synth.key_head_slice(inp, spec, b0, b0 + 32, 0, spec.Hk)
        o_ref, s_ref = oracle.gdn2_fwd(sl["q"], sl["k"], sl["v"], sl["a"], sl["A_log"], sl["erase"],
                                       sl["write"], S0=sl["S0"])
        accumulate_out(so, out[b0:b0 + 32], o_ref, b0=b0, bf16=True)
        accumulate_state(ss, S[b0:b0 + 32], s_ref, b0=b0)
    check_stats("out (16384 heads x 16 steps)", so, **BF16_DECODE_BOUNDS, rounded_tol=BF16_ROUNDED_TOL)
    check_stats("state (16384 heads)", ss, TOL["bf16"], head_tol=TOL["bf16"])


@pytest.mark.parametrize("dtype,Dk,Dv", [("f32", 128, 128), ("bf16", 128, 128), ("bf16", 64, 128)])
def test_ragged_persistent_tail(dtype, Dk, Dv):
    """B*Hv = 1072 heads: more than any resident grid (at most 4 work-groups on each of
    256 CUs) and not a multiple of 256, so the persistent loop walks several heads per
    work-group and ends on a partial sweep."""
    check(g2(B=67, T=3, Hk=4, Hv=16, Dk=Dk, Dv=Dv, dtype=dtype, seed=520 + Dk, init_state=True))
