"""GPU parity of the float32 Gated DeltaNet-2 chunked prefill (gdn2_chunk_fwd with
GDN_F32) against the float64 oracle (oracle.gdn2_fwd, the token-by-token recurrence
from raw logits).

float32 inputs, state and arithmetic: relative L2 <= 1e-5 over the whole output and
the whole final state, over every (sequence, value head) on its own and over every
(sequence, value head, 64-token chunk) of the output (measured at most 3.6e-7 on these
cases).  Every case prints its name and shape first.
"""
import math

import pytest
import torch

import oracle
import synth
from synth import GDNSpec, SLOW_DECAY
from tests.gpu_util import (TOL, Stats, accumulate_out, accumulate_state, assert_close, check_stats, log,
                            to_dev)

pytestmark = pytest.mark.gpu

F32_BOUNDS = dict(tol=TOL["f32"], head_tol=TOL["f32"], chunk_tol=TOL["f32"])


def gpu_gdn2(inp, scale: float = 1.0, **kw):
    import gated_deltanet_sequence_amd as gdn
    d = to_dev(inp)
    out, ST = gdn.gdn2_chunk_fwd(d["q"], d["k"], d["v"], d["a"], d["A_log"], d["erase"], d["write"],
                                 d["S0"], scale=scale, **kw)
    torch.cuda.synchronize()
    return out.cpu(), (None if ST is None else ST.cpu())


def full_check(spec: GDNSpec, scale: float = 1.0):
    log(f"[gdn2 f32] {spec}")
    inp = synth.make_inputs(spec)
    out, ST = gpu_gdn2(inp, scale=scale)
    assert out.dtype == torch.float32
    o_ref, s_ref = oracle.gdn2_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["A_log"], inp["erase"],
                                   inp["write"], S0=inp["S0"], scale=scale)
    so, ss = Stats(), Stats()
    accumulate_out(so, out, o_ref)
    accumulate_state(ss, ST, s_ref)
    check_stats("out", so, **F32_BOUNDS)
    check_stats("final_state", ss, tol=TOL["f32"], head_tol=TOL["f32"])
    return inp, out, ST


def g2(**kw) -> GDNSpec:
    return GDNSpec(variant="gdn2", dtype="f32", **kw)


def test_tiny_shape():
    """The tiny forward's shape (B=1, T=256, 2 key = 2 value heads, d=64) with GDN-2 gates."""
    full_check(g2(B=1, T=256, Hk=2, Hv=2, Dk=64, Dv=64, seed=700))


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_ragged_lengths(T):
    """One to four chunks and ragged tails."""
    full_check(g2(B=1, T=T, Hk=1, Hv=2, Dk=128, Dv=128, seed=710 + T, init_state=True))


@pytest.mark.parametrize("Dk,Dv", [(64, 64), (64, 128), (128, 64)])
def test_head_sizes(Dk, Dv):
    full_check(g2(B=1, T=257, Hk=1, Hv=2, Dk=Dk, Dv=Dv, seed=720 + Dk + Dv, init_state=True))


def test_batch_and_key_head_groups():
    """B=2 distinct sequences; 2 key heads shared by 2 value heads each; ragged T."""
    full_check(g2(B=2, T=130, Hk=2, Hv=4, Dk=128, Dv=128, seed=730, init_state=True))


def test_slow_decay_carries_state_across_chunks():
    full_check(g2(B=1, T=512, Hk=1, Hv=2, Dk=128, Dv=128, seed=740, init_state=True,
                  state_sigma=0.5, **SLOW_DECAY))


def test_wide_decay_range():
    """exp(A_log) from 1e-3 to 30 across channels: the in-chunk log decay reaches the
    hundreds, where each ratio needs the float64 prefix to stay exact in float32."""
    full_check(g2(B=1, T=300, Hk=1, Hv=2, Dk=128, Dv=128, seed=750, init_state=True,
                  state_sigma=0.3, a_log_lo=math.log(1e-3), a_log_hi=math.log(30.0)))


def test_scale():
    full_check(g2(B=1, T=150, Hk=1, Hv=2, Dk=128, Dv=128, seed=760, init_state=True), scale=0.0883883)


def test_reduces_to_scalar_gated_delta_rule():
    """A decay equal across channels and erase gate = write gate = beta: the float32
    GDN-2 path matches the float32 scalar-decay path (gdn_chunk_fwd, dt_bias = 0) and the
    scalar-decay oracle on the same problem, the reduction the update's definition gives."""
    import gated_deltanet_sequence_amd as gdn
    spec = g2(B=1, T=200, Hk=1, Hv=2, Dk=128, Dv=128, seed=770, init_state=True)
    log(f"[gdn2 f32 -> gdn f32] {spec}")
    inp = synth.make_inputs(spec)
    B, T, Hv, Dk, Dv = spec.B, spec.T, spec.Hv, spec.Dk, spec.Dv
    a_tok = inp["a"][..., 0].contiguous()      # [B,T,Hv], one logit per token shared by every channel
    b_tok = inp["erase"][..., 0].contiguous()
    A_row = inp["A_log"][:, 0].contiguous()
    inp2 = dict(inp)
    inp2["a"] = a_tok[..., None].expand(B, T, Hv, Dk).contiguous()
    inp2["erase"] = b_tok[..., None].expand(B, T, Hv, Dk).contiguous()
    inp2["write"] = b_tok[..., None].expand(B, T, Hv, Dv).contiguous()
    inp2["A_log"] = A_row[:, None].expand(Hv, Dk).contiguous()
    out, ST = gpu_gdn2(inp2)
    o_ref, s_ref = oracle.gdn_fwd(inp["q"], inp["k"], inp["v"], a_tok, b_tok, A_row, torch.zeros(Hv), S0=inp["S0"])
    assert_close("out (vs scalar-decay oracle)", out, o_ref, TOL["f32"])
    assert_close("final_state (vs scalar-decay oracle)", ST, s_ref, TOL["f32"])
    d = to_dev(inp)
    o1, s1 = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["a"][..., 0].contiguous(), d["erase"][..., 0].contiguous(),
                               d["A_log"][:, 0].contiguous(), torch.zeros(Hv, device="cuda"), d["S0"])
    torch.cuda.synchronize()
    assert_close("out (vs float32 gdn_chunk_fwd)", out, o1.cpu(), 2 * TOL["f32"])
    assert_close("final_state (vs float32 gdn_chunk_fwd)", ST, s1.cpu(), 2 * TOL["f32"])


def test_zero_initial_state_and_no_final_state():
    spec = g2(B=1, T=100, Hk=1, Hv=2, Dk=64, Dv=64, seed=780)
    log(f"[gdn2 f32 no final state] {spec}")
    inp = synth.make_inputs(spec)
    out, ST = gpu_gdn2(inp, output_final_state=False)
    assert ST is None
    o_ref, _ = oracle.gdn2_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["A_log"], inp["erase"],
                               inp["write"], S0=None)
    assert_close("out", out, o_ref, TOL["f32"])


def test_deterministic():
    spec = g2(B=1, T=150, Hk=1, Hv=2, Dk=128, Dv=128, seed=790, init_state=True)
    log(f"[gdn2 f32 determinism] {spec}")
    inp = synth.make_inputs(spec)
    o1, s1 = gpu_gdn2(inp)
    o2, s2 = gpu_gdn2(inp)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
