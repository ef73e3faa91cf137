"""The rule is linear in (v, S0): scaling both by a power of two scales outputs and final
state by the same factor exactly.  The bf16 chunked paths round value-sized operands to
float16, so their accuracy holds over a stated range of input magnitudes (include/gdn.h):
root mean square of v and of S0 in [2^-10, 2^10].  Inside it every case is gated at the
bf16 tolerance; outside it (2^-14, 2^-20) the results must stay finite and the error is
reported, not gated."""
import math

import pytest
import torch

import oracle
import synth
from synth import GDNSpec
from tests.gpu_util import TOL, assert_close, log, rel, to_dev

pytestmark = pytest.mark.gpu

IN_RANGE = [2.0 ** -10, 2.0 ** -6, 64.0, 2.0 ** 10]
OUT_OF_RANGE = [2.0 ** -14, 2.0 ** -20]


def scaled(inp, s):
    out = dict(inp)
    out["v"] = (inp["v"].float() * s).to(inp["v"].dtype)       # exact: power of two
    out["S0"] = inp["S0"] * s
    return out


def run_gdn(inp, s):
    import gated_deltanet_sequence_amd as gdn
    d = to_dev(scaled(inp, s))
    out, ST = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], d["S0"])
    torch.cuda.synchronize()
    return out.cpu(), ST.cpu()


def run_gdn2(inp, s):
    import gated_deltanet_sequence_amd as gdn
    d = to_dev(scaled(inp, s))
    out, ST = gdn.gdn2_chunk_fwd(d["q"], d["k"], d["v"], d["a"], d["A_log"], d["erase"], d["write"], d["S0"])
    torch.cuda.synchronize()
    return out.cpu(), ST.cpu()


SPEC = GDNSpec(B=1, T=200, Hk=1, Hv=4, Dk=128, Dv=128, dtype="bf16", seed=700, init_state=True,
               state_sigma=1.0)
SPEC2 = SPEC.with_(variant="gdn2", seed=701)


@pytest.fixture(scope="module")
def ref_gdn():
    inp = synth.make_inputs(SPEC)
    return inp, oracle.gdn_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"],
                               inp["dt_bias"], S0=inp["S0"])


@pytest.fixture(scope="module")
def ref_gdn2():
    inp = synth.make_inputs(SPEC2)
    return inp, oracle.gdn2_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["A_log"], inp["erase"],
                                inp["write"], S0=inp["S0"])


@pytest.mark.parametrize("s", IN_RANGE)
def test_prefill_scale_in_range(ref_gdn, s):
    inp, (o_ref, s_ref) = ref_gdn
    log(f"[prefill scale {s:g}] {SPEC}")
    out, ST = run_gdn(inp, s)
    # the oracle at scale 1, scaled by s (linearity; exact in float64 for a power of two)
    assert_close("out / s", out.double() / s, o_ref, TOL["bf16"])
    assert_close("final_state / s", ST.double() / s, s_ref, TOL["bf16"])


@pytest.mark.parametrize("s", IN_RANGE)
def test_gdn2_scale_in_range(ref_gdn2, s):
    inp, (o_ref, s_ref) = ref_gdn2
    log(f"[gdn2 scale {s:g}] {SPEC2}")
    out, ST = run_gdn2(inp, s)
    assert_close("out / s", out.double() / s, o_ref, TOL["bf16"])
    assert_close("final_state / s", ST.double() / s, s_ref, TOL["bf16"])


@pytest.mark.parametrize("s", OUT_OF_RANGE)
def test_scale_below_range_reported(ref_gdn, ref_gdn2, s):
    for name, (inp, (o_ref, s_ref)), fn in (("prefill", ref_gdn, run_gdn), ("gdn2", ref_gdn2, run_gdn2)):
        out, ST = fn(inp, s)
        assert torch.isfinite(out.float()).all() and torch.isfinite(ST).all()
        log(f"  {name} at scale {s:g} (outside the stated range): out rel-L2 "
            f"{rel(out.double() / s, o_ref):.3e}, final_state rel-L2 {rel(ST.double() / s, s_ref):.3e}")
