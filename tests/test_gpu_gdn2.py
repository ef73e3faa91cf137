"""GPU parity of the Gated DeltaNet-2 chunked prefill (gdn2_chunk_fwd) against the
float64 oracle (oracle.gdn2_fwd, the token-by-token recurrence from raw logits).

bfloat16 inputs, float32 state: relative L2 <= 2e-3 over the whole output and the
whole final state, separately.  Every case prints its name and shape first.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import GDNSpec, SLOW_DECAY, WORKLOADS
from tests.gpu_util import (BF16_BOUNDS, BF16_ROUNDED_TOL, TOL, Stats, accumulate_out, accumulate_state,
                            assert_close, check_stats, log, to_dev)

pytestmark = pytest.mark.gpu


def gpu_gdn2(inp, scale: float = 1.0, **kw):
    import gated_deltanet_sequence_amd as gdn
    d = to_dev(inp)
    out, ST = gdn.gdn2_chunk_fwd(d["q"], d["k"], d["v"], d["a"], d["A_log"], d["erase"], d["write"],
                                 d["S0"], scale=scale, **kw)
    torch.cuda.synchronize()
    return out.cpu(), (None if ST is None else ST.cpu())


def oracle_gdn2(inp, scale: float = 1.0):
    return oracle.gdn2_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["A_log"], inp["erase"],
                           inp["write"], S0=inp["S0"], scale=scale)


def full_check(spec: GDNSpec, scale: float = 1.0):
    log(f"[gdn2] {spec}")
    inp = synth.make_inputs(spec)
    out, ST = gpu_gdn2(inp, scale=scale)
    o_ref, s_ref = oracle_gdn2(inp, scale=scale)
    assert_close("out", out, o_ref, TOL["bf16"])
    assert_close("final_state", ST, s_ref, TOL["bf16"])
    return inp, out, ST


def g2(**kw) -> GDNSpec:
    return GDNSpec(variant="gdn2", dtype="bf16", **kw)


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 129, 200])
def test_ragged_lengths(T):
    """1 to 4 chunks (the scan stages its first two chunks before its loop) and ragged tails."""
    full_check(g2(B=1, T=T, Hk=1, Hv=2, Dk=128, Dv=128, seed=400 + T, init_state=True))


@pytest.mark.parametrize("Dk,Dv", [(64, 64), (64, 128), (128, 64)])
def test_head_sizes(Dk, Dv):
    full_check(g2(B=1, T=257, Hk=1, Hv=2, Dk=Dk, Dv=Dv, seed=410 + Dk + Dv, init_state=True))


def test_slow_decay_carries_state_across_chunks():
    """Per-channel decays near 1: the carried state and its per-channel decay dominate."""
    full_check(g2(B=1, T=512, Hk=2, Hv=4, Dk=128, Dv=128, seed=420, init_state=True,
                  state_sigma=0.5, **SLOW_DECAY))


def test_wide_decay_range():
    """exp(A_log) spread over 1e-3 .. 30 across channels: some channels keep their state
    over the whole sequence while others forget it within a token."""
    full_check(g2(B=1, T=300, Hk=1, Hv=2, Dk=128, Dv=128, seed=421, init_state=True,
                  state_sigma=0.3, a_log_lo=math.log(1e-3), a_log_hi=math.log(30.0)))


def test_batch_and_key_head_groups():
    """B=3 distinct sequences; 2 key heads shared by 4 value heads each."""
    full_check(g2(B=3, T=130, Hk=2, Hv=8, Dk=128, Dv=128, seed=430, init_state=True))


def test_zero_initial_state():
    full_check(g2(B=2, T=190, Hk=1, Hv=2, Dk=128, Dv=128, seed=431))


def test_scale():
    full_check(g2(B=1, T=100, Hk=1, Hv=2, Dk=128, Dv=128, seed=432, init_state=True),
               scale=1 / math.sqrt(128))


def test_in_place_final_state():
    spec = g2(B=2, T=150, Hk=1, Hv=2, Dk=128, Dv=128, seed=440, init_state=True)
    log(f"[gdn2 in-place] {spec}")
    inp = synth.make_inputs(spec)
    import gated_deltanet_sequence_amd as gdn
    d = to_dev(inp)
    S = d["S0"].clone()
    out, ST = gdn.gdn2_chunk_fwd(d["q"], d["k"], d["v"], d["a"], d["A_log"], d["erase"], d["write"],
                                 S, final_state=S)
    torch.cuda.synchronize()
    assert ST.data_ptr() == S.data_ptr()
    o_ref, s_ref = oracle_gdn2(inp)
    assert_close("out", out.cpu(), o_ref, TOL["bf16"])
    assert_close("final_state", S.cpu(), s_ref, TOL["bf16"])


def test_zero_length_copies_initial_state():
    spec = g2(B=2, T=0, Hk=1, Hv=2, Dk=128, Dv=128, seed=450, init_state=True)
    log(f"[gdn2 T=0] {spec}")
    inp = synth.make_inputs(spec)
    out, ST = gpu_gdn2(inp)
    assert out.numel() == 0
    assert torch.equal(ST, inp["S0"])


def test_reduces_to_scalar_gated_delta_rule():
    """A decay equal across channels and erase gate = write gate = beta: the GDN-2 kernels
    match the scalar-decay oracle (gated delta rule with dt_bias = 0) on the same problem,
    the reduction the update's definition gives."""
    spec = g2(B=1, T=200, Hk=1, Hv=2, Dk=128, Dv=128, seed=460, init_state=True)
    log(f"[gdn2 -> gdn] {spec}")
    inp = synth.make_inputs(spec)
    B, T, Hv, Dk, Dv = spec.B, spec.T, spec.Hv, spec.Dk, spec.Dv
    a_tok = inp["a"][..., 0].float()      # [B,T,Hv], one logit per token shared by every channel
    b_tok = inp["erase"][..., 0].float()
    A_row = inp["A_log"][:, 0].contiguous()
    inp2 = dict(inp)
    inp2["a"] = a_tok[..., None].expand(B, T, Hv, Dk).to(torch.bfloat16).contiguous()
    inp2["erase"] = b_tok[..., None].expand(B, T, Hv, Dk).to(torch.bfloat16).contiguous()
    inp2["write"] = b_tok[..., None].expand(B, T, Hv, Dv).to(torch.bfloat16).contiguous()
    inp2["A_log"] = A_row[:, None].expand(Hv, Dk).contiguous()
    out, ST = gpu_gdn2(inp2)
    o_ref, s_ref = oracle.gdn_fwd(inp["q"], inp["k"], inp["v"], a_tok, b_tok, A_row,
                                  torch.zeros(Hv), S0=inp["S0"])
    assert_close("out (vs scalar-decay oracle)", out, o_ref, TOL["bf16"])
    assert_close("final_state (vs scalar-decay oracle)", ST, s_ref, TOL["bf16"])


def test_deterministic():
    spec = g2(B=1, T=300, Hk=2, Hv=4, Dk=128, Dv=128, seed=470, init_state=True)
    log(f"[gdn2 determinism] {spec}")
    inp = synth.make_inputs(spec)
    o1, s1 = gpu_gdn2(inp)
    o2, s2 = gpu_gdn2(inp)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_gdn2_t8192_all_heads():
    """B=1, T=8192, 16 key / 64 value heads, d=128, bf16: the GDN-2 workload the bench
    times.  The oracle over every head and token (streamed over groups of four key heads)."""
    spec = WORKLOADS["gdn2_t8192"]
    log(f"[gdn2] {spec}")
    inp = synth.make_inputs(spec)
    out, ST = gpu_gdn2(inp)
    assert torch.isfinite(out.float()).all() and torch.isfinite(ST).all()
    G = spec.Hv // spec.Hk
    so, ss = Stats(), Stats()
    for hk0 in range(0, spec.Hk, 4):
        sl = synth.key_head_slice(inp, spec, 0, 1, hk0, hk0 + 4)
        o_ref, s_ref = oracle_gdn2(sl)
        h0, h1 = hk0 * G, (hk0 + 4) * G
        accumulate_out(so, out[:, :, h0:h1], o_ref, h0=h0, bf16=True)
        accumulate_state(ss, ST[:, h0:h1], s_ref, h0=h0)
    check_stats("out (64 heads)", so, **BF16_BOUNDS, rounded_tol=BF16_ROUNDED_TOL)
    check_stats("final_state (64 heads)", ss, TOL["bf16"], head_tol=TOL["bf16"])
