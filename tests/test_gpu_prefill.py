"""GPU parity of the chunked prefill (gdn_chunk_fwd) against the float64 oracle.

Tolerances (relative L2 over the whole tensor, outputs and final state
separately): 1e-5 for float32 inputs, 2e-3 for bfloat16 inputs with a float32
state.  Every case prints its name and shape before running on the GPU.
"""
import math

import numpy as np
import pytest
import torch

import synth
from synth import GDNSpec, SLOW_DECAY, WORKLOADS
from tests.gpu_util import (BF16_BOUNDS, BF16_ROUNDED_TOL, TOL, Stats, accumulate_out, accumulate_state,
                            assert_close, check_stats, gpu_prefill, log, oracle_prefill, to_dev)

pytestmark = pytest.mark.gpu


def full_check(spec: GDNSpec, scale: float = 1.0, tol=None):
    log(f"[prefill] {spec}")
    inp = synth.make_inputs(spec)
    out, ST = gpu_prefill(spec, inp, scale=scale)
    o_ref, s_ref = oracle_prefill(inp, scale=scale)
    tol = tol or TOL[spec.dtype]
    assert_close("out", out, o_ref, tol)
    assert_close("final_state", ST, s_ref, tol)
    return inp, out, ST


def test_tiny_f32_forward():
    """B=1, T=256, 2/2 heads, d=64, fp32, zero initial state."""
    full_check(WORKLOADS["tiny_f32"])


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_ragged_lengths_f32(T):
    full_check(GDNSpec(B=1, T=T, Hk=1, Hv=2, Dk=64, Dv=64, dtype="f32", seed=200 + T, init_state=True))


@pytest.mark.parametrize("Dk,Dv", [(64, 128), (128, 64), (128, 128)])
def test_head_sizes_f32(Dk, Dv):
    full_check(GDNSpec(B=1, T=192, Hk=1, Hv=2, Dk=Dk, Dv=Dv, dtype="f32", seed=210 + Dk + Dv,
                       init_state=True))


def test_slow_decay_f32_carries_state_across_chunks():
    """alpha ~ 0.97..0.999: the state survives many chunks, pinning the inter-chunk scan."""
    full_check(GDNSpec(B=1, T=512, Hk=2, Hv=4, Dk=128, Dv=128, dtype="f32", seed=220,
                       init_state=True, state_sigma=0.5, **SLOW_DECAY))


def test_batch_and_key_head_groups_f32():
    """B=3 distinct sequences; 2 key heads shared by 4 value heads each (distinct keys)."""
    full_check(GDNSpec(B=3, T=130, Hk=2, Hv=8, Dk=64, Dv=64, dtype="f32", seed=230, init_state=True))


def test_one_value_head_per_key_head_f32():
    full_check(GDNSpec(B=2, T=96, Hk=3, Hv=3, Dk=64, Dv=128, dtype="f32", seed=231, init_state=True))


def test_scale_f32():
    full_check(GDNSpec(B=1, T=100, Hk=1, Hv=2, Dk=128, Dv=64, dtype="f32", seed=232),
               scale=1 / math.sqrt(128))


def test_in_place_final_state_f32():
    spec = GDNSpec(B=2, T=150, Hk=1, Hv=2, Dk=64, Dv=64, dtype="f32", seed=240, init_state=True)
    log(f"[prefill in-place] {spec}")
    inp = synth.make_inputs(spec)
    import gated_deltanet_sequence_amd as gdn
    d = to_dev(inp)
    S = d["S0"].clone()
    out, ST = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], S,
                                final_state=S)
    torch.cuda.synchronize()
    assert ST.data_ptr() == S.data_ptr()
    o_ref, s_ref = oracle_prefill(inp)
    assert_close("out", out.cpu(), o_ref, TOL["f32"])
    assert_close("final_state", S.cpu(), s_ref, TOL["f32"])


def test_split_invariance_and_decode_handoff_f32():
    """Prefill of T tokens == prefill of T1, then T - T1 from its final state, then a decode
    step from that state equals one more token of the oracle."""
    spec = GDNSpec(B=2, T=201, Hk=1, Hv=2, Dk=64, Dv=64, dtype="f32", seed=250, init_state=True,
                   **SLOW_DECAY)
    log(f"[prefill split] {spec}")
    inp = synth.make_inputs(spec)
    import gated_deltanet_sequence_amd as gdn
    d = to_dev(inp)
    T1 = 77
    T = spec.T - 1
    sl = lambda x, a, b: x[:, a:b].contiguous()
    o1, s1 = gdn.gdn_chunk_fwd(sl(d["q"], 0, T1), sl(d["k"], 0, T1), sl(d["v"], 0, T1),
                               sl(d["a"], 0, T1), sl(d["b"], 0, T1), d["A_log"], d["dt_bias"], d["S0"])
    o2, s2 = gdn.gdn_chunk_fwd(sl(d["q"], T1, T), sl(d["k"], T1, T), sl(d["v"], T1, T),
                               sl(d["a"], T1, T), sl(d["b"], T1, T), d["A_log"], d["dt_bias"], s1)
    o3 = gdn.gdn_recurrent_step(d["q"][:, T].contiguous(), d["k"][:, T].contiguous(),
                                d["v"][:, T].contiguous(), d["a"][:, T].contiguous(),
                                d["b"][:, T].contiguous(), d["A_log"], d["dt_bias"], s2)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(inp)
    out = torch.cat([o1.cpu(), o2.cpu(), o3.cpu()[:, None]], dim=1)
    assert_close("out (split + step)", out, o_ref, TOL["f32"])
    assert_close("state after step", s2.cpu(), s_ref, TOL["f32"])


def test_zero_length_copies_initial_state():
    spec = GDNSpec(B=2, T=0, Hk=1, Hv=2, Dk=64, Dv=64, dtype="f32", seed=260, init_state=True)
    log(f"[prefill T=0] {spec}")
    inp = synth.make_inputs(spec)
    out, ST = gpu_prefill(spec, inp)
    assert out.numel() == 0
    assert torch.equal(ST, inp["S0"])
    spec0 = spec.with_(init_state=False)
    out, ST = gpu_prefill(spec0, synth.make_inputs(spec0))
    assert torch.count_nonzero(ST) == 0


def test_deterministic():
    spec = GDNSpec(B=1, T=300, Hk=2, Hv=8, Dk=128, Dv=128, dtype="bf16", seed=270, init_state=True)
    log(f"[prefill determinism] {spec}")
    inp = synth.make_inputs(spec)
    o1, s1 = gpu_prefill(spec, inp)
    o2, s2 = gpu_prefill(spec, inp)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_bf16_full_compare():
    """bf16 inputs, every element against the oracle: several chunks and a ragged tail."""
    full_check(GDNSpec(B=2, T=1000, Hk=4, Hv=16, Dk=128, Dv=128, dtype="bf16", seed=280,
                       init_state=True))


def test_bf16_persistent_units_with_ragged_tail():
    """1024 chunk-local units (2 x 16 key heads x 32 chunks) on a device holding 512 work-groups:
    each work-group walks two units and prefetches the second while computing the first, and
    some second units are the ragged last chunk (T = 2000 = 31 x 64 + 16), whose rows past the
    end are loaded from a clamped address and zeroed at conversion."""
    full_check(GDNSpec(B=2, T=2000, Hk=16, Hv=64, Dk=128, Dv=128, dtype="bf16", seed=285,
                       init_state=True))


def test_bf16_one_unit_per_work_group_with_ragged_tail():
    """2064 chunk-local units (16 key heads x 129 chunks, T = 8200 = 128 x 64 + 8): more than
    four per resident work-group, so each work-group takes one unit; the last chunk holds 8
    tokens."""
    full_check(GDNSpec(B=1, T=8200, Hk=16, Hv=64, Dk=128, Dv=128, dtype="bf16", seed=287,
                       init_state=True))


def test_f32_persistent_units_with_ragged_tail():
    """fp32, d_k = 128: 512 chunk-local units (2 x 16 key heads x 16 chunks) where the kernel's
    registers allow one work-group per CU, so each walks two units; T = 1000 leaves a ragged
    last chunk of 40 tokens."""
    full_check(GDNSpec(B=2, T=1000, Hk=16, Hv=32, Dk=128, Dv=64, dtype="f32", seed=286,
                       init_state=True))


# The bfloat16 path runs a different scan (float16 operands, role-split work-group
# with its own staging prologue for the first chunks): the same shape coverage.
@pytest.mark.parametrize("T", [1, 63, 64, 65, 129, 200])
def test_ragged_lengths_bf16(T):
    """1, 2, 3 and 4 chunks (the scan stages its first chunks before the loop) and ragged tails."""
    full_check(GDNSpec(B=1, T=T, Hk=1, Hv=2, Dk=128, Dv=128, dtype="bf16", seed=300 + T, init_state=True))


@pytest.mark.parametrize("Dk,Dv", [(64, 64), (64, 128), (128, 64)])
def test_head_sizes_bf16(Dk, Dv):
    full_check(GDNSpec(B=1, T=257, Hk=1, Hv=2, Dk=Dk, Dv=Dv, dtype="bf16", seed=310 + Dk + Dv,
                       init_state=True))


def test_batch_and_key_head_groups_bf16():
    """B=3 distinct sequences; 2 key heads shared by 4 value heads each."""
    full_check(GDNSpec(B=3, T=130, Hk=2, Hv=8, Dk=128, Dv=128, dtype="bf16", seed=330, init_state=True))


def test_scale_bf16():
    full_check(GDNSpec(B=1, T=100, Hk=1, Hv=2, Dk=128, Dv=128, dtype="bf16", seed=332),
               scale=1 / math.sqrt(128))


def test_in_place_final_state_bf16():
    spec = GDNSpec(B=2, T=150, Hk=1, Hv=2, Dk=128, Dv=128, dtype="bf16", seed=340, init_state=True)
    log(f"[prefill in-place] {spec}")
    inp = synth.make_inputs(spec)
    import gated_deltanet_sequence_amd as gdn
    d = to_dev(inp)
    S = d["S0"].clone()
    out, ST = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], S,
                                final_state=S)
    torch.cuda.synchronize()
    assert ST.data_ptr() == S.data_ptr()
    o_ref, s_ref = oracle_prefill(inp)
    assert_close("out", out.cpu(), o_ref, TOL["bf16"])
    assert_close("final_state", S.cpu(), s_ref, TOL["bf16"])


def test_bf16_slow_decay_reported():
    """Slow decay in bf16: the carried state dominates the output.  Gated at 2e-3 as well."""
    full_check(GDNSpec(B=1, T=512, Hk=2, Hv=4, Dk=128, Dv=128, dtype="bf16", seed=281,
                       init_state=True, **SLOW_DECAY))


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_many_heads_four_column_tiles(Dk, Dv):
    """More (sequence, value head, 32-column) units than CUs: the scan then gives each
    work-group 64 state columns (four state waves).  Ragged T, initial state, every head."""
    spec = GDNSpec(B=3, T=130, Hk=4, Hv=64, Dk=Dk, Dv=Dv, dtype="bf16", seed=360 + Dk + Dv, init_state=True)
    log(f"[prefill 64-column work-groups] {spec}")
    inp = synth.make_inputs(spec)
    out, ST = gpu_prefill(spec, inp)
    o_ref, s_ref = oracle_prefill(inp)
    so, ss = Stats(), Stats()
    accumulate_out(so, out, o_ref, bf16=True)
    accumulate_state(ss, ST, s_ref)
    check_stats("out", so, **BF16_BOUNDS, rounded_tol=BF16_ROUNDED_TOL)
    check_stats("final_state", ss, TOL["bf16"], head_tol=TOL["bf16"])


def test_qwen_shaped_prefill_t4096():
    """B=1, T=4096, 16 key / 64 value heads, d=128, bf16, zero state: the timed workload.
    The oracle over every head and token; whole-tensor, per-head and per-chunk errors."""
    spec = WORKLOADS["prefill_t4096"]
    log(f"[prefill] {spec}")
    inp = synth.make_inputs(spec)
    out, ST = gpu_prefill(spec, inp)
    assert torch.isfinite(out.float()).all() and torch.isfinite(ST).all()
    o_ref, s_ref = oracle_prefill(inp)
    so, ss = Stats(), Stats()
    accumulate_out(so, out, o_ref, bf16=True)
    accumulate_state(ss, ST, s_ref)
    check_stats("out (64 heads)", so, **BF16_BOUNDS, rounded_tol=BF16_ROUNDED_TOL)
    check_stats("final_state (64 heads)", ss, TOL["bf16"], head_tol=TOL["bf16"])


def test_long_context_prefill():
    """B=2, T=65536, 16/64 heads, d=128, bf16, initial state N(0, 0.02^2): every one of the
    128 (sequence, value head) pairs over all tokens, the oracle streamed over groups of four
    key heads (16 value heads) per sequence."""
    spec = WORKLOADS["prefill_long"]
    log(f"[prefill] {spec}")
    inp = synth.make_inputs(spec)
    out, ST = gpu_prefill(spec, inp)
    assert torch.isfinite(out.float()).all() and torch.isfinite(ST).all()
    G = spec.Hv // spec.Hk
    so, ss = Stats(), Stats()
    for b in range(spec.B):
        for hk0 in range(0, spec.Hk, 4):
            sl = synth.key_head_slice(inp, spec, b, b + 1, hk0, hk0 + 4)
            o_ref, s_ref = oracle_prefill(sl)
            h0, h1 = hk0 * G, (hk0 + 4) * G
            accumulate_out(so, out[b:b + 1, :, h0:h1], o_ref, b0=b, h0=h0, bf16=True)
            accumulate_state(ss, ST[b:b + 1, h0:h1], s_ref, b0=b, h0=h0)
            log(f"  sequence {b}, value heads {h0}..{h1 - 1}: running out rel-L2 {so.whole():.3e}")
    check_stats("out (128 heads)", so, **BF16_BOUNDS, rounded_tol=BF16_ROUNDED_TOL)
    check_stats("final_state (128 heads)", ss, TOL["bf16"], head_tol=TOL["bf16"])
