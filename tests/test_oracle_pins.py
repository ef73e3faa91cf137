"""Pins of the float64 oracle against what the pages and the mathematics fix.

None of these tests calls the GPU library.  Each pin is chosen so that a
plausible slip in the oracle (a dropped term, a wrong sign, a transposed state,
a wrong head map, read-out before the write, decay after the erase) fails at
least one of them.  The pins:

* gate closed forms (dingfen page, sections 9-10) against NumPy/SciPy routines;
* hand-worked examples worked from the rule by exact arithmetic (tests/golden/*.json),
  among them a Gated DeltaNet-2 example entered through the raw gate logits;
* alpha = 1, beta = 0 leaves the state unchanged (the identity transition);
* alpha = beta = 1 with a unit key writes v exactly at address k, and the
  interpolation identity of the dingfen page, section 7, for any beta;
* orthonormal keys reduce the delta rule to linear attention, whose outputs
  are the textbook product tril(Q K^T) V (dingfen page, section 3);
* beta = 0 gives pure exponential forgetting S_t = (prod alpha) S_0 (section 9);
* brute force: the state as an explicit product of d_k x d_k transition
  matrices (rainlin page, gated delta rule formula);
* the pages' chunkwise WY form (zhichai page) reproduces the token loop;
* GDN-2 with b = w = beta 1 and D = alpha I reduces to GDN (zhichai page,
  section "退化兼容性"), both through explicit gates and through the raw logits
  (channel-constant logits against the GDN gates with dt_bias = 0).
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
from oracle import wy_chunk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_problem(rng, B=2, T=7, Hk=1, Hv=2, Dk=5, Dv=3, unit_keys=True):
    q = rng.standard_normal((B, T, Hk, Dk))
    k = rng.standard_normal((B, T, Hk, Dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, Hv, Dv))
    g = -rng.uniform(0.0, 1.5, size=(B, T, Hv))
    beta = rng.uniform(0.0, 1.0, size=(B, T, Hv))
    return q, k, v, g, beta


# ---------------------------------------------------------------- gates

def test_softplus_matches_library_and_closed_forms(oracle_lib):
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), rel=0, abs=1e-16)
    for x in [-700.0, -40.0, -30.0, -1.5, -1e-8, 0.0, 1e-8, 0.3, 2.0, 30.0, 40.0, 700.0]:
        assert oracle.softplus(x) == pytest.approx(float(np.logaddexp(0.0, x)), rel=1e-15, abs=1e-300)
    # softplus(x) - softplus(-x) = x (log(1+e^x) - log(1+e^-x) = x)
    for x in [0.1, 3.0, 25.0]:
        assert oracle.softplus(x) - oracle.softplus(-x) == pytest.approx(x, rel=1e-14)


def test_sigmoid_matches_library(oracle_lib):
    assert oracle.sigmoid(0.0) == 0.5
    for x in [-50.0, -3.0, -0.1, 0.7, 4.0, 50.0]:
        assert oracle.sigmoid(x) == pytest.approx(float(expit(x)), rel=1e-15)
    assert oracle.sigmoid(-math.inf) == 0.0 and oracle.sigmoid(math.inf) == 1.0


def test_gdn_gates_closed_form(oracle_lib):
    rng = np.random.default_rng(1)
    Hv = 4
    a = rng.standard_normal((3, 5, Hv)) * 10
    a[0, 0] = [30.0, -30.0, 0.0, 5.0]
    b = rng.standard_normal((3, 5, Hv)) * 3
    A_log = np.array([0.0, math.log(16.0), -1.0, 0.5])
    dt_bias = np.array([0.0, 0.0, -0.7, 0.9])
    g, beta = oracle.gdn_gates(a, b, A_log, dt_bias)
    want_g = -np.exp(A_log) * np.logaddexp(0.0, a + dt_bias)
    np.testing.assert_allclose(g, want_g, rtol=1e-14, atol=0)
    np.testing.assert_allclose(beta, expit(b), rtol=1e-15, atol=0)
    # A_log = 0, x = 0 gives g = -ln 2 (alpha = 1/2); large x: g ~ -exp(A_log) x
    assert g[0, 0, 2] != 0 and g[0, 0, 0] == pytest.approx(-30.0 - math.log1p(math.exp(-30.0)), rel=1e-15)
    assert np.all(g <= 0) and np.all((beta > 0) & (beta < 1))


def test_gdn2_gates_closed_form(oracle_lib):
    rng = np.random.default_rng(2)
    Hv, Dk, Dv = 2, 3, 4
    a = rng.standard_normal((2, 3, Hv, Dk)) * 4
    e = rng.standard_normal((2, 3, Hv, Dk))
    w = rng.standard_normal((2, 3, Hv, Dv))
    A_log = rng.uniform(0, math.log(16), size=(Hv, Dk))
    g, eb, wb = oracle.gdn2_gates(a, A_log, e, w)
    np.testing.assert_allclose(g, -np.exp(A_log) * np.logaddexp(0.0, a), rtol=1e-14)
    np.testing.assert_allclose(eb, expit(e), rtol=1e-15)
    np.testing.assert_allclose(wb, expit(w), rtol=1e-15)


# ---------------------------------------------------------------- worked examples

def test_hand_worked_gdn_example(oracle_lib):
    fx = json.load(open(os.path.join(GOLDEN, "hand_worked_gdn.json")))
    i = {k: np.array(v, dtype=np.float64) for k, v in fx["inputs"].items()}
    out, ST = oracle.gdn_fwd(i["q"], i["k"], i["v"], i["a"], i["b"], i["A_log"], i["dt_bias"])
    tol = fx["tolerance_abs"]
    np.testing.assert_allclose(out, np.array(fx["expected"]["out"]), rtol=0, atol=tol)
    np.testing.assert_allclose(ST, np.array(fx["expected"]["final_state"]), rtol=0, atol=tol)


def test_hand_worked_gdn2_example(oracle_lib):
    fx = json.load(open(os.path.join(GOLDEN, "hand_worked_gdn2.json")))
    i = {k: np.array(v, dtype=np.float64) for k, v in fx["inputs"].items()}
    out, ST = oracle.gdn2_core(i["q"], i["k"], i["v"], i["g"], i["eb"], i["wb"], S0=i["S0"])
    tol = fx["tolerance_abs"]
    np.testing.assert_allclose(out, np.array(fx["expected"]["out"]), rtol=0, atol=tol)
    np.testing.assert_allclose(ST, np.array(fx["expected"]["final_state"]), rtol=0, atol=tol)


def test_hand_worked_gdn2_raw_logit_example(oracle_lib):
    """The GDN-2 forward from raw logits (decay logit a with A_log per key channel, erase and
    write logits): gates and recurrence together, against values worked by hand."""
    fx = json.load(open(os.path.join(GOLDEN, "hand_worked_gdn2_logits.json")))
    i = {k: np.array(v, dtype=np.float64) for k, v in fx["inputs"].items()}
    out, ST = oracle.gdn2_fwd(i["q"], i["k"], i["v"], i["a"], i["A_log"], i["erase"], i["write"],
                              S0=i["S0"])
    tol = fx["tolerance_abs"]
    np.testing.assert_allclose(out, np.array(fx["expected"]["out"]), rtol=0, atol=tol)
    np.testing.assert_allclose(ST, np.array(fx["expected"]["final_state"]), rtol=0, atol=tol)


# ---------------------------------------------------------------- special cases

def test_identity_when_alpha_one_beta_zero(oracle_lib):
    rng = np.random.default_rng(3)
    q, k, v, g, beta = _rand_problem(rng)
    S0 = rng.standard_normal((2, 2, 5, 3))
    out, ST = oracle.gdn_core(q, k, v, np.zeros_like(g), np.zeros_like(beta), S0=S0, scale=0.5)
    np.testing.assert_array_equal(ST, S0)
    # o_t = scale * S0^T q_t, value head hv reading key head 0
    want = 0.5 * np.einsum("bhkv,btk->bthv", S0, q[:, :, 0])
    np.testing.assert_allclose(out, want, rtol=1e-13, atol=1e-13)


def test_exact_write_with_unit_key(oracle_lib):
    """alpha = beta = 1, |k| = 1: after the step, S_t^T k_t = v_t."""
    rng = np.random.default_rng(4)
    Dk, Dv, T = 6, 4, 9
    q, k, v, _, _ = _rand_problem(rng, B=1, T=T, Hk=1, Hv=1, Dk=Dk, Dv=Dv)
    S = rng.standard_normal((1, 1, Dk, Dv))
    for t in range(T):
        _, S = oracle.gdn_core(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1],
                               np.zeros((1, 1, 1)), np.ones((1, 1, 1)), S0=S)
        np.testing.assert_allclose(S[0, 0].T @ k[0, t, 0], v[0, t, 0], rtol=0, atol=1e-13)


def test_interpolation_identity_any_beta(oracle_lib):
    """S_t^T k = (1 - beta |k|^2) alpha S_{t-1}^T k + beta |k|^2 v (dingfen page, section 7,
    with the decay applied first)."""
    rng = np.random.default_rng(5)
    Dk, Dv, T = 5, 3, 12
    q, k, v, g, beta = _rand_problem(rng, B=1, T=T, Hk=1, Hv=1, Dk=Dk, Dv=Dv, unit_keys=False)
    S = rng.standard_normal((1, 1, Dk, Dv))
    for t in range(T):
        kt, vt, al, be = k[0, t, 0], v[0, t, 0], math.exp(g[0, t, 0]), beta[0, t, 0]
        prev = S[0, 0].T @ kt
        _, S = oracle.gdn_core(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], g[:, t:t + 1],
                               beta[:, t:t + 1], S0=S)
        nk = kt @ kt
        want = (1 - be * nk) * al * prev + be * nk * vt
        np.testing.assert_allclose(S[0, 0].T @ kt, want, rtol=1e-12, atol=1e-12)


def test_orthonormal_keys_reduce_to_linear_attention(oracle_lib):
    """With orthonormal keys nothing is erased, so the rule is S_t = S_{t-1} + k v^T and
    o_t = sum_{i<=t} (q_t . k_i) v_i = (tril(Q K^T) V)_t; each key retrieves its value."""
    rng = np.random.default_rng(6)
    Dk, Dv, T = 8, 5, 6
    Kmat, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    keys = Kmat[:, :T].T                         # T orthonormal rows
    q = rng.standard_normal((1, T, 1, Dk))
    k = keys[None, :, None, :]
    v = rng.standard_normal((1, T, 1, Dv))
    out, ST = oracle.gdn_core(q, k, v, np.zeros((1, T, 1)), np.ones((1, T, 1)))
    Q, V = q[0, :, 0], v[0, :, 0]
    want = np.tril(Q @ keys.T) @ V
    np.testing.assert_allclose(out[0, :, 0], want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ST[0, 0], keys.T @ V, rtol=1e-12, atol=1e-12)
    for j in range(T):
        np.testing.assert_allclose(ST[0, 0].T @ keys[j], V[j], rtol=1e-12, atol=1e-12)


def test_pure_forgetting_when_beta_zero(oracle_lib):
    rng = np.random.default_rng(7)
    q, k, v, g, _ = _rand_problem(rng, B=1, T=10, Hk=1, Hv=1)
    S0 = rng.standard_normal((1, 1, 5, 3))
    out, ST = oracle.gdn_core(q, k, v, g, np.zeros_like(g), S0=S0)
    cum = np.exp(np.cumsum(g[0, :, 0]))
    np.testing.assert_allclose(ST[0, 0], cum[-1] * S0[0, 0], rtol=1e-13)
    for t in range(10):
        np.testing.assert_allclose(out[0, t, 0], cum[t] * S0[0, 0].T @ q[0, t, 0], rtol=1e-12, atol=1e-14)


def _brute_force(q, k, v, g, beta, S0):
    """S_t = P_t S_{t-1} + beta_t k_t v_t^T with P_t = alpha_t (I - beta_t k_t k_t^T) as an
    explicit d_k x d_k matrix; all earlier steps composed by matrix products."""
    T, Dk = q.shape
    outs, S = [], S0.copy()
    for t in range(T):
        P = math.exp(g[t]) * (np.eye(Dk) - beta[t] * np.outer(k[t], k[t]))
        S = P @ S + beta[t] * np.outer(k[t], v[t])
        outs.append(S.T @ q[t])
    return np.array(outs), S


def test_brute_force_rank_one_products(oracle_lib):
    rng = np.random.default_rng(8)
    q, k, v, g, beta = _rand_problem(rng, B=2, T=11, Hk=2, Hv=4, Dk=5, Dv=3, unit_keys=False)
    S0 = rng.standard_normal((2, 4, 5, 3))
    out, ST = oracle.gdn_core(q, k, v, g, beta, S0=S0, scale=1.0)
    for b in range(2):
        for hv in range(4):
            hk = hv // 2                                      # value head -> key head map
            o, s = _brute_force(q[b, :, hk], k[b, :, hk], v[b, :, hv], g[b, :, hv], beta[b, :, hv],
                                S0[b, hv])
            np.testing.assert_allclose(out[b, :, hv], o, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(ST[b, hv], s, rtol=1e-12, atol=1e-12)


def test_brute_force_closed_product_form(oracle_lib):
    """S_T = prod_t P_t S_0 + sum_t (prod_{s>t} P_s) beta_t k_t v_t^T, formed as one sum."""
    rng = np.random.default_rng(9)
    T, Dk, Dv = 6, 4, 3
    q, k, v, g, beta = _rand_problem(rng, B=1, T=T, Hk=1, Hv=1, Dk=Dk, Dv=Dv, unit_keys=False)
    S0 = rng.standard_normal((1, 1, Dk, Dv))
    _, ST = oracle.gdn_core(q, k, v, g, beta, S0=S0)
    P = [math.exp(g[0, t, 0]) * (np.eye(Dk) - beta[0, t, 0] * np.outer(k[0, t, 0], k[0, t, 0]))
         for t in range(T)]

    def prod(a, b_):  # P_{b-1} ... P_a
        M = np.eye(Dk)
        for s in range(a, b_):
            M = P[s] @ M
        return M
    want = prod(0, T) @ S0[0, 0]
    for t in range(T):
        want = want + prod(t + 1, T) @ (beta[0, t, 0] * np.outer(k[0, t, 0], v[0, t, 0]))
    np.testing.assert_allclose(ST[0, 0], want, rtol=1e-12, atol=1e-12)


def test_decode_one_pass_readout(oracle_lib):
    """o = alpha S^T q + (k . q) delta: the step's read-out from the old state."""
    rng = np.random.default_rng(10)
    B, Hk, Hv, Dk, Dv = 3, 2, 4, 6, 5
    q = rng.standard_normal((B, Hk, Dk)); k = rng.standard_normal((B, Hk, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, Hv, Dv)); a = rng.standard_normal((B, Hv)); b = rng.standard_normal((B, Hv))
    A_log = rng.uniform(0, math.log(16), Hv); dt_bias = rng.uniform(-1, 1, Hv)
    S = rng.standard_normal((B, Hv, Dk, Dv)) * 0.02
    out, Snew = oracle.gdn_step(q, k, v, a, b, A_log, dt_bias, S)
    g, beta = oracle.gdn_gates(a, b, A_log, dt_bias)
    for bb in range(B):
        for hv in range(Hv):
            hk = hv // 2
            al = math.exp(g[bb, hv])
            kv = al * S[bb, hv].T @ k[bb, hk]
            d = beta[bb, hv] * (v[bb, hv] - kv)
            want = al * S[bb, hv].T @ q[bb, hk] + (k[bb, hk] @ q[bb, hk]) * d
            np.testing.assert_allclose(out[bb, hv], want, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(Snew[bb, hv], al * S[bb, hv] + np.outer(k[bb, hk], d),
                                       rtol=1e-12, atol=1e-15)


def test_sequences_and_heads_are_independent(oracle_lib):
    """Each (sequence, value head) is its own recurrence: solving it alone gives the same."""
    rng = np.random.default_rng(11)
    q, k, v, g, beta = _rand_problem(rng, B=3, T=8, Hk=2, Hv=6, Dk=4, Dv=3)
    out, ST = oracle.gdn_core(q, k, v, g, beta)
    for b in range(3):
        for hv in range(6):
            hk = hv // 3
            o1, s1 = oracle.gdn_core(q[b:b + 1, :, hk:hk + 1], k[b:b + 1, :, hk:hk + 1],
                                     v[b:b + 1, :, hv:hv + 1], g[b:b + 1, :, hv:hv + 1],
                                     beta[b:b + 1, :, hv:hv + 1])
            np.testing.assert_array_equal(out[b, :, hv], o1[0, :, 0])
            np.testing.assert_array_equal(ST[b, hv], s1[0, 0])


def test_scale_is_a_pure_multiplier(oracle_lib):
    rng = np.random.default_rng(12)
    q, k, v, g, beta = _rand_problem(rng)
    o1, s1 = oracle.gdn_core(q, k, v, g, beta, scale=1.0)
    o2, s2 = oracle.gdn_core(q, k, v, g, beta, scale=1 / math.sqrt(5))
    np.testing.assert_allclose(o2, o1 / math.sqrt(5), rtol=1e-14)
    np.testing.assert_array_equal(s1, s2)


# ---------------------------------------------------------------- chunk form

@pytest.mark.parametrize("T,C", [(200, 64), (64, 64), (1, 64), (37, 16)])
def test_wy_chunk_form_matches_token_loop(oracle_lib, T, C):
    rng = np.random.default_rng(13 + T)
    q, k, v, g, beta = _rand_problem(rng, B=1, T=T, Hk=1, Hv=2, Dk=16, Dv=24)
    S0 = rng.standard_normal((1, 2, 16, 24)) * 0.1
    o_ref, s_ref = oracle.gdn_core(q, k, v, g, beta, S0=S0)
    o_wy, s_wy = wy_chunk.gdn_chunk_fwd(q, k, v, g, beta, S0=S0, C=C)
    np.testing.assert_allclose(o_wy, o_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(s_wy, s_ref, rtol=1e-10, atol=1e-12)


def test_wy_chunk_form_with_strong_decay(oracle_lib):
    """Cumulative log decays far below the float range of 1/gamma still give the token loop."""
    rng = np.random.default_rng(14)
    q, k, v, g, beta = _rand_problem(rng, B=1, T=130, Hk=1, Hv=1, Dk=8, Dv=8)
    g = g * 40.0                                    # ~ -30 per token, ~ -1900 per chunk
    o_ref, s_ref = oracle.gdn_core(q, k, v, g, beta)
    o_wy, s_wy = wy_chunk.gdn_chunk_fwd(q, k, v, g, beta, C=64)
    np.testing.assert_allclose(o_wy, o_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(s_wy, s_ref, rtol=1e-10, atol=1e-300)


# ---------------------------------------------------------------- GDN-2

def test_gdn2_reduces_to_gdn(oracle_lib):
    rng = np.random.default_rng(15)
    B, T, Hk, Hv, Dk, Dv = 2, 9, 1, 2, 5, 4
    q, k, v, g, beta = _rand_problem(rng, B=B, T=T, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv)
    S0 = rng.standard_normal((B, Hv, Dk, Dv))
    o1, s1 = oracle.gdn_core(q, k, v, g, beta, S0=S0)
    g2 = np.repeat(g[..., None], Dk, axis=-1)
    eb = np.repeat(beta[..., None], Dk, axis=-1)
    wb = np.repeat(beta[..., None], Dv, axis=-1)
    o2, s2 = oracle.gdn2_core(q, k, v, g2, eb, wb, S0=S0)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s2, s1, rtol=1e-12, atol=1e-13)


def test_gdn2_raw_logits_reduce_to_gdn(oracle_lib):
    """Channel-constant raw logits: a[t,h,c] = a[t,h], A_log[h,c] = A_log[h] and erase = write
    logits = b[t,h] make the GDN-2 gates D = alpha 1, b = w = beta 1, so gdn2_fwd must equal
    gdn_fwd (whose gates are pinned by closed forms) with dt_bias = 0."""
    rng = np.random.default_rng(19)
    B, T, Hk, Hv, Dk, Dv = 2, 11, 1, 3, 4, 5
    q = rng.standard_normal((B, T, Hk, Dk))
    k = rng.standard_normal((B, T, Hk, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, Hv, Dv))
    a = rng.standard_normal((B, T, Hv)) * 2
    b = rng.standard_normal((B, T, Hv)) * 2
    A_log = rng.uniform(-1.0, math.log(16.0), size=Hv)
    S0 = rng.standard_normal((B, Hv, Dk, Dv))
    o1, s1 = oracle.gdn_fwd(q, k, v, a, b, A_log, np.zeros(Hv), S0=S0, scale=0.7)
    o2, s2 = oracle.gdn2_fwd(q, k, v, np.repeat(a[..., None], Dk, -1), np.repeat(A_log[:, None], Dk, -1),
                             np.repeat(b[..., None], Dk, -1), np.repeat(b[..., None], Dv, -1),
                             S0=S0, scale=0.7)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s2, s1, rtol=1e-12, atol=1e-13)
    # a channel-varying decay must not reduce (the pin would catch a gate that ignores c)
    A2 = np.repeat(A_log[:, None], Dk, -1).copy()
    A2[:, 0] += 1.0
    o3, _ = oracle.gdn2_fwd(q, k, v, np.repeat(a[..., None], Dk, -1), A2, np.repeat(b[..., None], Dk, -1),
                            np.repeat(b[..., None], Dv, -1), S0=S0, scale=0.7)
    assert oracle.rel_l2(o3, o1) > 1e-3


def test_gdn2_brute_force(oracle_lib):
    """S_t = (I - k e^T) D S_{t-1} + k z^T with explicit d_k x d_k matrices."""
    rng = np.random.default_rng(16)
    T, Dk, Dv = 8, 5, 3
    q = rng.standard_normal((1, T, 1, Dk)); k = rng.standard_normal((1, T, 1, Dk))
    v = rng.standard_normal((1, T, 1, Dv))
    g = -rng.uniform(0, 1.5, (1, T, 1, Dk)); eb = rng.uniform(0, 1, (1, T, 1, Dk))
    wb = rng.uniform(0, 1, (1, T, 1, Dv))
    S0 = rng.standard_normal((1, 1, Dk, Dv))
    out, ST = oracle.gdn2_core(q, k, v, g, eb, wb, S0=S0)
    S = S0[0, 0].copy()
    for t in range(T):
        kt, e = k[0, t, 0], eb[0, t, 0] * k[0, t, 0]
        S = (np.eye(Dk) - np.outer(kt, e)) @ np.diag(np.exp(g[0, t, 0])) @ S \
            + np.outer(kt, wb[0, t, 0] * v[0, t, 0])
        np.testing.assert_allclose(out[0, t, 0], S.T @ q[0, t, 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ST[0, 0], S, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("T,C", [(70, 16), (64, 64), (5, 4)])
def test_gdn2_wy_chunk_form_matches_token_loop(oracle_lib, T, C):
    rng = np.random.default_rng(17 + T)
    Dk, Dv = 6, 5
    q = rng.standard_normal((1, T, 1, Dk)); k = rng.standard_normal((1, T, 1, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, T, 2, Dv))
    g = -rng.uniform(0, 3.0, (1, T, 2, Dk)); eb = rng.uniform(0, 1, (1, T, 2, Dk))
    wb = rng.uniform(0, 1, (1, T, 2, Dv))
    S0 = rng.standard_normal((1, 2, Dk, Dv)) * 0.1
    o_ref, s_ref = oracle.gdn2_core(q, k, v, g, eb, wb, S0=S0)
    o_wy, s_wy = wy_chunk.gdn2_chunk_fwd(q, k, v, g, eb, wb, S0=S0, C=C)
    np.testing.assert_allclose(o_wy, o_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(s_wy, s_ref, rtol=1e-10, atol=1e-12)


def test_gdn2_fwd_composes_gates_and_core(oracle_lib):
    rng = np.random.default_rng(18)
    B, T, Hk, Hv, Dk, Dv = 1, 6, 1, 2, 4, 3
    q = rng.standard_normal((B, T, Hk, Dk)); k = rng.standard_normal((B, T, Hk, Dk))
    v = rng.standard_normal((B, T, Hv, Dv)); a = rng.standard_normal((B, T, Hv, Dk))
    e = rng.standard_normal((B, T, Hv, Dk)); w = rng.standard_normal((B, T, Hv, Dv))
    A_log = rng.uniform(0, math.log(16), (Hv, Dk))
    o1, s1 = oracle.gdn2_fwd(q, k, v, a, A_log, e, w)
    g, eb, wb = oracle.gdn2_gates(a, A_log, e, w)
    o2, s2 = oracle.gdn2_core(q, k, v, g, eb, wb)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


# ---------------------------------------------------------------- planted mistakes

def test_pins_catch_planted_mistakes(oracle_lib):
    """Variants of the recurrence with a classic slip must fail the brute-force pin."""
    rng = np.random.default_rng(19)
    T, Dk, Dv = 6, 4, 3
    q, k, v, g, beta = _rand_problem(rng, B=1, T=T, Hk=1, Hv=1, Dk=Dk, Dv=Dv, unit_keys=False)
    S0 = rng.standard_normal((Dk, Dv))
    o_bf, s_bf = _brute_force(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0], S0)

    def variant(kind):
        S = S0.copy(); outs = []
        for t in range(T):
            kt, vt, qt = k[0, t, 0], v[0, t, 0], q[0, t, 0]
            al, be = math.exp(g[0, t, 0]), beta[0, t, 0]
            if kind == "decay_after_erase":          # the undecayed-error variant
                d = be * (vt - S.T @ kt); S = al * S + np.outer(kt, d)
            else:
                S = al * S; d = be * (vt - S.T @ kt)
                if kind == "sign":
                    d = be * (vt + S.T @ kt)
                if kind == "readout_before_write":
                    outs.append(S.T @ qt)
                S = S + np.outer(kt, d)
            if kind != "readout_before_write":
                outs.append(S.T @ qt)
        return np.array(outs), S

    for kind in ["decay_after_erase", "sign", "readout_before_write"]:
        o, s = variant(kind)
        assert not np.allclose(o, o_bf, rtol=1e-6, atol=1e-9), kind


# ---------------------------------------------------------------- gated RMSNorm epilogue

def test_hand_worked_gated_rmsnorm(oracle_lib):
    fx = json.load(open(os.path.join(GOLDEN, "hand_worked_gated_rmsnorm.json")))
    i = fx["inputs"]
    x, z, w = (np.array(i[n], dtype=np.float64) for n in ("x", "z", "w"))
    for name, gate in (("sigmoid", oracle.GATE_SIGMOID), ("silu", oracle.GATE_SILU)):
        y = oracle.gated_rmsnorm(x, z, w, i["eps"], gate)
        np.testing.assert_allclose(y, np.array(fx["expected"][name]), rtol=0, atol=fx["tolerance_abs"])


def test_gated_rmsnorm_against_library_rms_norm(oracle_lib):
    """With the sigmoid gate saturated at 1 (z = 60) the epilogue is a plain RMSNorm:
    torch.nn.functional.rms_norm in float64, with eps."""
    import torch
    rng = np.random.default_rng(41)
    x = rng.standard_normal((37, 128)) * 3.0
    w = rng.uniform(0.5, 1.5, size=128)
    for eps in (1e-6, 0.3):
        y = oracle.gated_rmsnorm(x, np.full_like(x, 60.0), w, eps, oracle.GATE_SIGMOID)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(w), eps).numpy()
        np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_gated_rmsnorm_gate_and_scale_identities(oracle_lib):
    """SiLU(z) = z sigmoid(z) relates the two gates; with eps = 0 the result does not depend
    on the scale of x; a constant row normalises to its sign."""
    rng = np.random.default_rng(42)
    x = rng.standard_normal((9, 64))
    z = rng.standard_normal((9, 64)) * 2
    w = rng.uniform(-1, 1, size=64)
    y_sig = oracle.gated_rmsnorm(x, z, w, 0.0, oracle.GATE_SIGMOID)
    y_silu = oracle.gated_rmsnorm(x, z, w, 0.0, oracle.GATE_SILU)
    np.testing.assert_allclose(y_silu, y_sig * z, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(oracle.gated_rmsnorm(37.5 * x, z, w, 0.0, oracle.GATE_SILU), y_silu,
                               rtol=1e-13, atol=1e-14)
    c = np.full((2, 64), -2.5)
    np.testing.assert_allclose(oracle.gated_rmsnorm(c, z[:2], w, 0.0, oracle.GATE_SIGMOID),
                               -w * expit(z[:2]), rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- causal conv1d prologue

def test_hand_worked_causal_conv1d(oracle_lib):
    fx = json.load(open(os.path.join(GOLDEN, "hand_worked_causal_conv1d.json")))
    i = {k: np.array(v, dtype=np.float64) for k, v in fx["inputs"].items()}
    y, st = oracle.causal_conv1d(i["x"], i["w"], state=i["state"], silu=False)
    tol = fx["tolerance_abs"]
    np.testing.assert_allclose(y, np.array(fx["expected"]["y"]), rtol=0, atol=tol)
    np.testing.assert_allclose(st, np.array(fx["expected"]["state_out"]), rtol=0, atol=tol)
    y, _ = oracle.causal_conv1d(i["x"], i["w"], state=i["state"], silu=True)
    assert abs(y[0, 0, 0] - fx["expected"]["y0_silu"]) <= tol


def test_causal_conv1d_against_library_conv(oracle_lib):
    """A zero state is torch's depthwise conv1d (groups = channels) with K-1 zeros of left
    padding, then SiLU; a bias adds per channel."""
    import torch
    rng = np.random.default_rng(51)
    B, T, C, K = 2, 37, 24, 4
    x = rng.standard_normal((B, T, C))
    w = rng.standard_normal((C, K))
    bias = rng.standard_normal(C)
    y, st = oracle.causal_conv1d(x, w, bias=bias, silu=True)
    xt = torch.from_numpy(x).transpose(1, 2)                      # [B, C, T]
    ref = torch.nn.functional.conv1d(xt, torch.from_numpy(w)[:, None, :], torch.from_numpy(bias),
                                     padding=K - 1, groups=C)[..., :T]
    ref = torch.nn.functional.silu(ref).transpose(1, 2).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(st, x[:, T - (K - 1):], rtol=0, atol=0)


def test_causal_conv1d_split_invariance(oracle_lib):
    """Running T tokens in pieces, each starting from the previous piece's state (including
    pieces shorter than K-1 and single-token steps), equals one pass."""
    rng = np.random.default_rng(52)
    B, T, C, K = 2, 23, 16, 4
    x = rng.standard_normal((B, T, C))
    w = rng.standard_normal((C, K))
    s0 = rng.standard_normal((B, K - 1, C))
    y_all, st_all = oracle.causal_conv1d(x, w, state=s0)
    st, ys, t = s0, [], 0
    for n in (1, 2, 1, 7, 1, 1, 10):
        y, st = oracle.causal_conv1d(x[:, t:t + n], w, state=st)
        ys.append(y)
        t += n
    assert t == T
    np.testing.assert_allclose(np.concatenate(ys, axis=1), y_all, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(st, st_all, rtol=0, atol=0)
