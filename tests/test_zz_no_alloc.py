"""gdn_chunk_fwd_noalloc (the prefill with the library's own device scratch) against
gdn_chunk_fwd (caller workspace): the same kernels on the same inputs must give identical
outputs and final states.  Two calls in a row share the scratch, the second on a smaller
input, so stale contents of the first call would show; an fp32 call follows (its workspace
layout differs); dims beyond the scratch are rejected."""
import pytest
import torch

import synth
from synth import GDNSpec, WORKLOADS
from tests.gpu_util import TOL, assert_close, log, oracle_prefill, to_dev

pytestmark = pytest.mark.gpu


def both(spec):
    import gated_deltanet_sequence_amd as gdn
    inp = synth.make_inputs(spec)
    d = to_dev(inp)
    args = (d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], d["S0"])
    o1, s1 = gdn.gdn_chunk_fwd(*args)
    # preallocated outputs: the no-allocation call itself allocates nothing
    o2 = torch.full_like(o1, float("nan"))
    s2 = torch.full_like(s1, float("nan"))
    gdn.gdn_chunk_fwd_noalloc(*args, out=o2, final_state=s2)
    torch.cuda.synchronize()
    return inp, (o1.cpu(), s1.cpu()), (o2.cpu(), s2.cpu())


@pytest.mark.parametrize("spec", [
    WORKLOADS["prefill_t4096"],                                                   # 86 MB of scratch
    GDNSpec(B=2, T=200, Hk=2, Hv=8, Dk=128, Dv=128, dtype="bf16", seed=900, init_state=True),
    GDNSpec(B=1, T=130, Hk=1, Hv=2, Dk=64, Dv=128, dtype="f32", seed=901, init_state=True),
    GDNSpec(B=1, T=65, Hk=1, Hv=1, Dk=128, Dv=64, dtype="bf16", seed=902),
], ids=["t4096", "small_bf16", "f32", "ragged"])
def test_noalloc_matches_workspace_entry(spec):
    log(f"[noalloc] {spec}")
    inp, (o1, s1), (o2, s2) = both(spec)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    if spec.T <= 256:
        o_ref, s_ref = oracle_prefill(inp)
        assert_close("out", o2, o_ref, TOL[spec.dtype])
        assert_close("final_state", s2, s_ref, TOL[spec.dtype])


def test_noalloc_rejects_dims_beyond_its_scratch():
    import gated_deltanet_sequence_amd as gdn
    spec = GDNSpec(B=1, T=8192, Hk=16, Hv=64, Dk=128, Dv=128, dtype="bf16", seed=903)
    q = torch.zeros((1, spec.T, 16, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((1, spec.T, 64, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((1, spec.T, 64), device="cuda")
    h = torch.zeros(64, device="cuda")
    with pytest.raises(gdn.GDNError, match="scratch"):
        gdn.gdn_chunk_fwd_noalloc(q, q, v, g, g, h, h)
