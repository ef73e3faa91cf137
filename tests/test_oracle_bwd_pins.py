"""Pins of the float64 oracle's Gated DeltaNet-2 backward (oracle.gdn2_bwd).

The backward is pinned by central finite differences of the forward oracle
(oracle.gdn2_fwd), which is itself pinned in test_oracle_pins.py: for
L = sum(d_out * out) + sum(d_ST * S_T), every gradient element the backward
returns must equal (L(x + h) - L(x - h)) / 2h for that input element.  The
finite differences use only the forward, so a dropped term, a wrong sign or a
transposed operand anywhere in the reverse pass fails here.  None of these
tests calls the GPU library.
"""
import math

import numpy as np
import pytest

import oracle

NAMES = ["q", "k", "v", "a", "A_log", "erase", "write", "S0"]
GRAD = {"q": "dq", "k": "dk", "v": "dv", "a": "da", "A_log": "dA_log", "erase": "d_erase",
        "write": "d_write", "S0": "dS0"}


def _problem(rng, B, T, Hk, Hv, Dk, Dv):
    x = {
        "q": rng.standard_normal((B, T, Hk, Dk)),
        "k": rng.standard_normal((B, T, Hk, Dk)) * 0.7,
        "v": rng.standard_normal((B, T, Hv, Dv)),
        "a": rng.standard_normal((B, T, Hv, Dk)),
        "A_log": rng.uniform(math.log(0.05), math.log(2.0), (Hv, Dk)),
        "erase": rng.standard_normal((B, T, Hv, Dk)),
        "write": rng.standard_normal((B, T, Hv, Dv)),
        "S0": rng.standard_normal((B, Hv, Dk, Dv)) * 0.5,
    }
    dout = rng.standard_normal((B, T, Hv, Dv))
    dST = rng.standard_normal((B, Hv, Dk, Dv))
    return x, dout, dST


def _loss(x, dout, dST, scale):
    o, s = oracle.gdn2_fwd(x["q"], x["k"], x["v"], x["a"], x["A_log"], x["erase"], x["write"],
                           S0=x["S0"], scale=scale)
    return float(np.sum(o * dout) + (np.sum(s * dST) if dST is not None else 0.0))


def _check(x, dout, dST, scale, rng, per_tensor=None, h=1e-5):
    grads = oracle.gdn2_bwd(x["q"], x["k"], x["v"], x["a"], x["A_log"], x["erase"], x["write"],
                            dout, S0=x["S0"], d_ST=dST, scale=scale)
    for name in NAMES:
        g = grads[GRAD[name]]
        assert g.shape == x[name].shape, name
        n = x[name].size
        idx = np.arange(n) if per_tensor is None or n <= per_tensor else rng.choice(n, per_tensor, replace=False)
        fd = np.empty(len(idx))
        for m, i in enumerate(idx):
            xp = {kk: vv.copy() for kk, vv in x.items()}
            xm = {kk: vv.copy() for kk, vv in x.items()}
            xp[name].flat[i] += h
            xm[name].flat[i] -= h
            fd[m] = (_loss(xp, dout, dST, scale) - _loss(xm, dout, dST, scale)) / (2 * h)
        got = g.reshape(-1)[idx]
        np.testing.assert_allclose(got, fd, rtol=2e-6, atol=2e-7 * max(1.0, np.abs(fd).max()),
                                   err_msg=name)
        assert np.abs(fd).max() > 1e-3, name  # the check is not vacuous
    return grads


def test_bwd_matches_finite_differences_small(oracle_lib):
    """Every element of every gradient, two value heads sharing one key head, scale != 1."""
    rng = np.random.default_rng(70)
    x, dout, dST = _problem(rng, B=1, T=5, Hk=1, Hv=2, Dk=3, Dv=4)
    _check(x, dout, dST, 0.7, rng)


def test_bwd_matches_finite_differences_across_segments(oracle_lib):
    """T = 70 crosses the backward's stretch of 64 recomputed states; B = 2, two key heads
    of two value heads each; sampled elements of every gradient."""
    rng = np.random.default_rng(71)
    x, dout, dST = _problem(rng, B=2, T=70, Hk=2, Hv=4, Dk=2, Dv=3)
    _check(x, dout, dST, 1.0, rng, per_tensor=40)


def test_bwd_without_final_state_gradient(oracle_lib):
    """d_ST = None means a zero final-state gradient; S0 = None means a zero initial state."""
    rng = np.random.default_rng(72)
    x, dout, dST = _problem(rng, B=1, T=6, Hk=1, Hv=1, Dk=3, Dv=2)
    g1 = oracle.gdn2_bwd(x["q"], x["k"], x["v"], x["a"], x["A_log"], x["erase"], x["write"], dout)
    g2 = oracle.gdn2_bwd(x["q"], x["k"], x["v"], x["a"], x["A_log"], x["erase"], x["write"], dout,
                         S0=np.zeros_like(x["S0"]), d_ST=np.zeros_like(dST))
    for kk in g1:
        np.testing.assert_array_equal(g1[kk], g2[kk])
    x["S0"] = np.zeros_like(x["S0"])
    _check(x, dout, None, 1.0, rng)


def test_bwd_state_only_gradient_is_the_transition_adjoint(oracle_lib):
    """With d_out = 0, dS0 = (prod of transitions)^T d_ST: the state map S_T = P S0 + c is
    affine in S0 with P = F_T ... F_1, F_t = (I - k e^T) diag(D) (zhichai page, the
    Gated Delta Rule-2 transition), so its adjoint is P^T d_ST."""
    rng = np.random.default_rng(73)
    B, T, Hk, Hv, Dk, Dv = 1, 9, 1, 1, 4, 3
    x, dout, dST = _problem(rng, B, T, Hk, Hv, Dk, Dv)
    gr = oracle.gdn2_bwd(x["q"], x["k"], x["v"], x["a"], x["A_log"], x["erase"], x["write"],
                         np.zeros_like(dout), S0=x["S0"], d_ST=dST)
    g, eb, _ = oracle.gdn2_gates(x["a"], x["A_log"], x["erase"], x["write"])
    P = np.eye(Dk)
    for t in range(T):
        kt = x["k"][0, t, 0]
        F = (np.eye(Dk) - np.outer(kt, eb[0, t, 0] * kt)) @ np.diag(np.exp(g[0, t, 0]))
        P = F @ P
    np.testing.assert_allclose(gr["dS0"][0, 0], P.T @ dST[0, 0], rtol=1e-12, atol=1e-13)
    assert np.abs(gr["dq"]).max() == 0.0  # q only reaches the output
