"""GPU parity of the causal conv1d + SiLU prologue (gdn_causal_conv1d) against the
float64 oracle (oracle.causal_conv1d): the q, k, v split of the output and the new
conv state.  Relative L2: 1e-5 for float32, 2e-3 for bfloat16; the state holds copies
of inputs and must match exactly."""
import pytest
import torch

import oracle
import synth
from tests.gpu_util import TOL, assert_close, log

pytestmark = pytest.mark.gpu


def split(y, Hk, Hv, Dk, Dv):
    B, T, _ = y.shape
    qk = Hk * Dk
    return (y[..., :qk].reshape(B, T, Hk, Dk), y[..., qk:2 * qk].reshape(B, T, Hk, Dk),
            y[..., 2 * qk:].reshape(B, T, Hv, Dv))


def check(B, T, Hk, Hv, Dk, Dv, dtype, seed, bias=True, state=True, act="silu"):
    import gated_deltanet_sequence_amd as gdn
    C = 2 * Hk * Dk + Hv * Dv
    log(f"[conv1d] B={B} T={T} Hk={Hk} Hv={Hv} Dk={Dk} Dv={Dv} {dtype} bias={bias} state={state} {act}")
    x, w, b, s = synth.make_conv_inputs(B, T, C, dtype, seed, bias=bias, state=state)
    dev = lambda t: None if t is None else t.cuda()
    q, k, v, so = gdn.gdn_causal_conv1d(dev(x), dev(w), dev(b), dev(s), Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv,
                                        activation=act)
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.causal_conv1d(x, w, bias=b, state=s, silu=act == "silu")
    if T:
        for name, got, ref in zip("qkv", (q, k, v), split(torch.from_numpy(y_ref), Hk, Hv, Dk, Dv)):
            assert_close(name, got.cpu(), ref, TOL[dtype])
    assert torch.equal(so.cpu().double(), torch.from_numpy(s_ref)), "conv state"


@pytest.mark.parametrize("T", [1, 2, 3, 15, 16, 17, 63, 64, 65, 100, 130])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lengths(T, dtype):
    """Waves of 8 tokens handing their last rows to the next wave, work-groups of 64 tokens
    loading their own halo: a partial first block, exact blocks and work-groups, ragged tails
    inside and across work-groups; T < 3 takes part of the new state from the old one."""
    check(2, T, 2, 4, 64, 64, dtype, seed=700 + T)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_channels_not_a_multiple_of_the_work_group(dtype):
    """C = 192: a work-group covers 256 channels, so a quarter of its lanes hold none."""
    check(2, 70, 1, 1, 64, 64, dtype, seed=730)


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 128), (128, 64)])
def test_head_sizes_bf16(Dk, Dv):
    check(1, 50, 2, 8, Dk, Dv, "bf16", seed=710 + Dk + Dv)


def test_no_bias_no_state_no_activation_f32():
    check(3, 40, 1, 2, 64, 64, "f32", seed=720, bias=False, state=False, act="none")


def test_zero_length_copies_the_state():
    check(2, 0, 1, 2, 64, 64, "bf16", seed=721)


def test_qwen_shaped_prefill_bf16():
    """B=1, T=4096, 16 key / 64 value heads, d=128: C = 12,288 channels."""
    check(1, 4096, 16, 64, 128, 128, "bf16", seed=722)


def test_decode_steps_in_place_match_one_pass():
    """A prefill of 37 tokens, then 12 decode steps (T = 1) updating the state in place, equal
    the oracle's single pass over the 49 tokens."""
    import gated_deltanet_sequence_amd as gdn
    B, Hk, Hv, Dk, Dv = 3, 2, 4, 64, 128
    C = 2 * Hk * Dk + Hv * Dv
    x, w, b, s0 = synth.make_conv_inputs(B, 49, C, "f32", seed=723)
    log(f"[conv1d prefill + steps] B={B} C={C}")
    xd, wd, bd = x.cuda(), w.cuda(), b.cuda()
    q, k, v, st = gdn.gdn_causal_conv1d(xd[:, :37].contiguous(), wd, bd, s0.cuda(), Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv)
    ys = [torch.cat([q.flatten(2), k.flatten(2), v.flatten(2)], dim=-1)]
    for t in range(37, 49):
        q, k, v, st2 = gdn.gdn_causal_conv1d(xd[:, t:t + 1].contiguous(), wd, bd, st, Hk=Hk, Hv=Hv, Dk=Dk,
                                             Dv=Dv, conv_state_out=st)
        assert st2.data_ptr() == st.data_ptr()
        ys.append(torch.cat([q.flatten(2), k.flatten(2), v.flatten(2)], dim=-1))
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.causal_conv1d(x, w, bias=b, state=s0)
    assert_close("outputs (prefill + 12 steps)", torch.cat(ys, dim=1).cpu(), y_ref, TOL["f32"])
    assert torch.equal(st.cpu().double(), torch.from_numpy(s_ref))
