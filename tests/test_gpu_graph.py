"""HIP graph capture of the decode step and of the chunked prefill.

The library allocates nothing, synchronises nothing and records no memset, so
a caller can capture its calls in a graph.  Each test captures one call, then
replays the graph several times, copying new inputs into the captured buffers
between replays (ordinary eager work on the same stream), and checks every
replay bit for bit against the same call made eagerly on the same inputs.
"""
import dataclasses

import pytest
import torch

import synth
from synth import GDNSpec
from tests.gpu_util import log, to_dev

pytestmark = pytest.mark.gpu


def capture(fn):
    """Capture fn() in a CUDA/HIP graph after one warm-up call on a side stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(warmup=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res = fn(warmup=False)
    return g, res


def test_decode_step_replays_match_eager():
    import gated_deltanet_sequence_amd as gdn
    spec = GDNSpec(B=4, T=5, Hk=4, Hv=16, Dk=128, Dv=128, dtype="bf16", seed=700, init_state=True)
    log(f"[graph decode] {spec}")
    d = to_dev(synth.make_inputs(spec))
    tok = lambda name, t: d[name][:, t].contiguous()
    names = ("q", "k", "v", "a", "b")
    static = {n: tok(n, 0).clone() for n in names}
    S_graph, S_eager = d["S0"].clone(), d["S0"].clone()

    def step(warmup):
        S = S_graph.clone() if warmup else S_graph  # the warm-up must not advance the state
        return gdn.gdn_recurrent_step(static["q"], static["k"], static["v"], static["a"], static["b"],
                                      d["A_log"], d["dt_bias"], S)

    g, out_graph = capture(step)
    assert torch.equal(S_graph, d["S0"])  # capture itself runs nothing
    for t in range(spec.T):
        for n in names:
            static[n].copy_(tok(n, t))
        g.replay()
        out_eager = gdn.gdn_recurrent_step(tok("q", t), tok("k", t), tok("v", t), tok("a", t), tok("b", t),
                                           d["A_log"], d["dt_bias"], S_eager)
        torch.cuda.synchronize()
        assert torch.equal(out_graph, out_eager), f"output of replay {t}"
        assert torch.equal(S_graph, S_eager), f"state after replay {t}"


def test_prefill_replays_match_eager():
    import gated_deltanet_sequence_amd as gdn
    spec = GDNSpec(B=2, T=200, Hk=4, Hv=16, Dk=128, Dv=128, dtype="bf16", seed=701, init_state=True)
    log(f"[graph prefill] {spec}")
    names = ("q", "k", "v", "a", "b", "S0")
    inputs = [to_dev(synth.make_inputs(dataclasses.replace(spec, seed=spec.seed + i))) for i in range(3)]
    static = {n: inputs[0][n].clone() for n in names}
    A_log, dt_bias = inputs[0]["A_log"], inputs[0]["dt_bias"]

    def run(warmup):
        return gdn.gdn_chunk_fwd(static["q"], static["k"], static["v"], static["a"], static["b"], A_log,
                                 dt_bias, static["S0"])

    g, (out_graph, ST_graph) = capture(run)
    for rep in range(4):
        cur = inputs[rep % 3]
        for n in names:
            static[n].copy_(cur[n])
        g.replay()
        out_eager, ST_eager = gdn.gdn_chunk_fwd(cur["q"], cur["k"], cur["v"], cur["a"], cur["b"], A_log,
                                                dt_bias, cur["S0"])
        torch.cuda.synchronize()
        assert torch.equal(out_graph, out_eager), f"output of replay {rep}"
        assert torch.equal(ST_graph, ST_eager), f"final state of replay {rep}"


def test_gdn2_forward_and_backward_replays_match_eager():
    import gated_deltanet_sequence_amd as gdn
    spec = GDNSpec(variant="gdn2", B=1, T=150, Hk=2, Hv=4, Dk=128, Dv=128, dtype="bf16", seed=702,
                   init_state=True)
    log(f"[graph gdn2] {spec}")
    names = ("q", "k", "v", "a", "erase", "write", "S0", "d_out", "d_ST")

    def make(i):
        s = dataclasses.replace(spec, seed=spec.seed + i)
        d = to_dev(synth.make_inputs(s))
        d.update(to_dev(synth.make_grad_inputs(s)))
        return d

    inputs = [make(i) for i in range(3)]
    static = {n: inputs[0][n].clone() for n in names}
    A_log = inputs[0]["A_log"]

    def fwd(x):
        return gdn.gdn2_chunk_fwd(x["q"], x["k"], x["v"], x["a"], A_log, x["erase"], x["write"], x["S0"])

    def bwd(x):
        return gdn.gdn2_chunk_bwd(x["q"], x["k"], x["v"], x["a"], A_log, x["erase"], x["write"], x["S0"],
                                  x["d_out"], x["d_ST"])

    g, (fo, fs, grads) = capture(lambda warmup: (*fwd(static), bwd(static)))
    for rep in range(4):
        cur = inputs[rep % 3]
        for n in names:
            static[n].copy_(cur[n])
        g.replay()
        eo, es = fwd(cur)
        eg = bwd(cur)
        torch.cuda.synchronize()
        assert torch.equal(fo, eo) and torch.equal(fs, es), f"forward of replay {rep}"
        assert sorted(grads) == sorted(eg)
        for name in grads:
            assert torch.equal(grads[name], eg[name]), f"{name} of replay {rep}"
