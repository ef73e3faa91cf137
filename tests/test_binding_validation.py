"""The binding rejects, before any library call reaches the GPU, tensors a kernel would
misuse: host tensors (their addresses would be dereferenced on the device), tensors on
another device, and caller-supplied outputs, workspaces or gradient buffers of the wrong
shape, dtype or size.  CPU only: every check fires before a kernel is enqueued."""
import pytest
import torch

import gated_deltanet_sequence_amd as gdn

B, T, Hk, Hv, Dk, Dv = 1, 8, 1, 2, 64, 64
bf, f32 = torch.bfloat16, torch.float32


def prefill_args():
    return dict(q=torch.zeros(B, T, Hk, Dk, dtype=bf), k=torch.zeros(B, T, Hk, Dk, dtype=bf),
                v=torch.zeros(B, T, Hv, Dv, dtype=bf), a=torch.zeros(B, T, Hv), b=torch.zeros(B, T, Hv),
                A_log=torch.zeros(Hv), dt_bias=torch.zeros(Hv))


def gdn2_args():
    return dict(q=torch.zeros(B, T, Hk, Dk, dtype=bf), k=torch.zeros(B, T, Hk, Dk, dtype=bf),
                v=torch.zeros(B, T, Hv, Dv, dtype=bf), a=torch.zeros(B, T, Hv, Dk, dtype=bf),
                A_log=torch.zeros(Hv, Dk), erase=torch.zeros(B, T, Hv, Dk, dtype=bf),
                write=torch.zeros(B, T, Hv, Dv, dtype=bf))


def test_prefill_rejects_host_tensors():
    with pytest.raises(ValueError, match="GPU tensors"):
        gdn.gdn_chunk_fwd(**prefill_args())


@pytest.mark.parametrize("name,bad,exc", [
    ("out", torch.zeros(B, T, Hv, Dv, dtype=f32), TypeError),        # float32 out for bf16 q
    ("out", torch.zeros(B, T, Hv, Dv + 1, dtype=bf), ValueError),     # too large a row
    ("final_state", torch.zeros(B, Hv, Dk, Dv, dtype=bf), TypeError),
    ("final_state", torch.zeros(B, Hv, Dk, 1), ValueError),
    ("initial_state", torch.zeros(B, Hv + 1, Dk, Dv), ValueError),
    ("workspace", torch.zeros(16, dtype=torch.uint8), ValueError),   # too small
])
def test_prefill_rejects_bad_outputs(name, bad, exc):
    kw = prefill_args()
    kw[name] = bad
    with pytest.raises(exc):
        gdn.gdn_chunk_fwd(**kw)


@pytest.mark.parametrize("name,bad,exc", [
    ("a", torch.zeros(B, T, Hv), ValueError),
    ("a", torch.zeros(B, T, Hv, Dk), TypeError),
    ("v", torch.zeros(B, T, Hv, Dv + 1, dtype=bf), ValueError),
    ("A_log", torch.zeros(Hv), ValueError),
])
def test_prefill_rejects_bad_inputs(name, bad, exc):
    kw = prefill_args()
    if name == "a" and bad.dim() == 4:
        kw = gdn2_args()
        kw["a"] = bad
        with pytest.raises(exc):
            gdn.gdn2_chunk_fwd(**kw)
        return
    kw[name] = bad
    with pytest.raises(exc):
        gdn.gdn_chunk_fwd(**kw)


def test_gdn2_rejects_host_tensors_and_bad_outputs():
    with pytest.raises(ValueError, match="GPU tensors"):
        gdn.gdn2_chunk_fwd(**gdn2_args())
    with pytest.raises(TypeError):
        gdn.gdn2_chunk_fwd(**gdn2_args(), out=torch.zeros(B, T, Hv, Dv, dtype=f32))
    with pytest.raises(ValueError):
        gdn.gdn2_chunk_fwd(**gdn2_args(), final_state=torch.zeros(B, Hv, Dk, Dv + 2))


def test_bwd2_rejects_bad_grads():
    kw = gdn2_args()
    d_out = torch.zeros(B, T, Hv, Dv, dtype=bf)
    with pytest.raises(ValueError, match="GPU tensors"):
        gdn.gdn2_chunk_bwd(**kw, initial_state=None, d_out=d_out)
    good = {"dq": torch.zeros(B, T, Hk, Dk), "dk": torch.zeros(B, T, Hk, Dk), "dv": torch.zeros(B, T, Hv, Dv),
            "da": torch.zeros(B, T, Hv, Dk), "d_erase": torch.zeros(B, T, Hv, Dk),
            "d_write": torch.zeros(B, T, Hv, Dv), "dA_log": torch.zeros(Hv, Dk),
            "d_initial_state": torch.zeros(B, Hv, Dk, Dv)}
    for name, bad, exc in [("dq", torch.zeros(B, T, Hv, Dk), ValueError),
                           ("dA_log", torch.zeros(Hv, Dk, dtype=bf), TypeError),
                           ("dv", torch.zeros(B, T, Hv, Dv + 1), ValueError)]:
        g = dict(good)
        g[name] = bad
        with pytest.raises(exc):
            gdn.gdn2_chunk_bwd(**kw, initial_state=None, d_out=d_out, grads=g)
    g = dict(good)
    del g["dk"]
    with pytest.raises(ValueError, match="missing"):
        gdn.gdn2_chunk_bwd(**kw, initial_state=None, d_out=d_out, grads=g)
    with pytest.raises(TypeError):
        gdn.gdn2_chunk_bwd(**kw, initial_state=None, d_out=torch.zeros(B, T, Hv, Dv), grads=good)


def test_steps_reject_host_tensors_and_bad_outputs():
    q = torch.zeros(B, Hk, Dk, dtype=bf)
    kw = dict(q=q, k=q.clone(), v=torch.zeros(B, Hv, Dv, dtype=bf), a=torch.zeros(B, Hv),
              b=torch.zeros(B, Hv), A_log=torch.zeros(Hv), dt_bias=torch.zeros(Hv),
              state=torch.zeros(B, Hv, Dk, Dv))
    with pytest.raises(ValueError, match="GPU tensors"):
        gdn.gdn_recurrent_step(**kw)
    with pytest.raises(TypeError):
        gdn.gdn_recurrent_step(**kw, out=torch.zeros(B, Hv, Dv))
    kw["state"] = torch.zeros(B, Hv, Dk, Dv, dtype=bf)
    with pytest.raises(TypeError):
        gdn.gdn_recurrent_step(**kw)
    kw2 = dict(q=q, k=q.clone(), v=torch.zeros(B, Hv, Dv, dtype=bf), a=torch.zeros(B, Hv, Dk, dtype=bf),
               A_log=torch.zeros(Hv, Dk), erase=torch.zeros(B, Hv, Dk, dtype=bf),
               write=torch.zeros(B, Hv, Dv, dtype=bf), state=torch.zeros(B, Hv, Dk, Dv))
    with pytest.raises(ValueError, match="GPU tensors"):
        gdn.gdn2_recurrent_step(**kw2)
    with pytest.raises(ValueError):
        gdn.gdn2_recurrent_step(**kw2, out=torch.zeros(B, Hv, Dv + 1, dtype=bf))


def test_norm_and_conv_reject_host_tensors_and_bad_outputs():
    x = torch.zeros(4, 64, dtype=bf)
    with pytest.raises(ValueError, match="GPU tensors"):
        gdn.gdn_gated_rmsnorm(x, x.clone(), torch.ones(64))
    with pytest.raises(TypeError):
        gdn.gdn_gated_rmsnorm(x, x.clone(), torch.ones(64), out=torch.zeros(4, 64))
    C = 2 * Hk * Dk + Hv * Dv
    xc = torch.zeros(B, T, C, dtype=bf)
    kw = dict(Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv)
    with pytest.raises(ValueError, match="GPU tensors"):
        gdn.gdn_causal_conv1d(xc, torch.zeros(C, 4), **kw)
    with pytest.raises(ValueError):
        gdn.gdn_causal_conv1d(xc, torch.zeros(C, 4), q=torch.zeros(B, T, Hk, Dk + 1, dtype=bf), **kw)
    with pytest.raises(TypeError):
        gdn.gdn_causal_conv1d(xc, torch.zeros(C, 4), v=torch.zeros(B, T, Hv, Dv), **kw)
