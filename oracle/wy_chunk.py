"""The pages' chunkwise (WY) form of the gated delta rule, NumPy float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  This is a second,
independent route to the same outputs as the token loop in ``gdn_oracle.c``;
the tests check that the two agree to rounding, which pins both.

Source: zhichai.net, "Gated DeltaNet-2" digest, section "高效训练：WY 算法依然成立"
(decay-normalised state, WY auxiliaries, chunk output and chunk state).  In the
page's notation, inside a chunk with cumulative decay gamma_r (product of the
per-token decays D_1..D_r of that chunk):

* kbar_r = k_r / gamma_r,  ebar_r = gamma_r (.) (b_r (.) k_r),  z_r = w_r (.) v_r;
* A = (I + tril(Ebar Kbar^T, -1))^{-1},  Y = A Ebar,  U = A Z;
* O[n] = Q_gamma S[n] + A_qk (U - Y S[n]);
* S[n+1] = Diag(gamma_C) S[n] + K_tail^T (U - Y S[n]).

The page leaves Q_gamma, A_qk and K_tail undefined.  Reading adopted (it is the
one that makes the chunk form reproduce the token recurrence exactly): row r of
Q_gamma is gamma_r (.) q_r; A_qk = tril(Q_gamma Kbar^T, 0) including the
diagonal; row i of K_tail is (gamma_C / gamma_i) (.) k_i.  The state is stored
as S[d_k][d_v], so "Diag(gamma) S" scales rows (key channels).

Scalar GDN is the special case D_t = alpha_t I, b_t = beta_t 1, w_t = beta_t 1
(same page, section "退化兼容性").

Every product of a gamma with a 1/gamma is formed as exp(G_r - G_i) from the
cumulative log decay G, which is the same number without the overflow of
1/gamma in finite precision.
"""
from __future__ import annotations

import numpy as np


def _tri_inverse_unit_lower(L: np.ndarray) -> np.ndarray:
    """(I + L)^{-1} for strictly lower-triangular L, by forward substitution."""
    n = L.shape[0]
    X = np.zeros((n, n))
    for c in range(n):
        x = np.zeros(n)
        for r in range(n):
            x[r] = (1.0 if r == c else 0.0) - L[r, :r] @ x[:r]
        X[:, c] = x
    return X


def chunk_fwd_head(q, k, v, g, eb, wb, S0, C: int):
    """One (sequence, value head) pair through the WY chunk form.

    q, k : [T, Dk]; v : [T, Dv]; g : [T, Dk] log decay per key channel;
    eb : [T, Dk] erase gate; wb : [T, Dv] write gate; S0 : [Dk, Dv].
    Returns out [T, Dv] (unscaled read-out S_t^T q_t) and S_T [Dk, Dv].
    """
    T, Dk = q.shape
    Dv = v.shape[1]
    S = np.array(S0, dtype=np.float64, copy=True)
    out = np.zeros((T, Dv))
    for t0 in range(0, T, C):
        t1 = min(T, t0 + C)
        n = t1 - t0
        Q, K, V = q[t0:t1], k[t0:t1], v[t0:t1]
        G = np.cumsum(g[t0:t1], axis=0)            # log gamma_r, inclusive, restarts per chunk
        E = eb[t0:t1] * K                           # e_r = b_r (.) k_r
        Z = wb[t0:t1] * V                           # z_r = w_r (.) v_r
        # (Ebar Kbar^T)[r,i] = sum_c exp(G[r,c] - G[i,c]) e[r,c] k[i,c]
        # (Q_gamma Kbar^T)[r,i] = sum_c exp(G[r,c] - G[i,c]) q[r,c] k[i,c]
        EK = np.zeros((n, n))
        QK = np.zeros((n, n))
        for r in range(n):
            for i in range(r + 1):
                ratio = np.exp(G[r] - G[i])
                EK[r, i] = np.sum(ratio * E[r] * K[i])
                QK[r, i] = np.sum(ratio * Q[r] * K[i])
        A = _tri_inverse_unit_lower(np.tril(EK, -1))
        Ebar = np.exp(G) * E                         # gamma_r (.) e_r
        Y = A @ Ebar
        U = A @ Z
        Qg = np.exp(G) * Q                           # Q_gamma
        Aqk = np.tril(QK, 0)
        Vnew = U - Y @ S
        out[t0:t1] = Qg @ S + Aqk @ Vnew
        Ktail = np.exp(G[-1][None, :] - G) * K        # (gamma_C / gamma_i) (.) k_i
        S = np.exp(G[-1])[:, None] * S + Ktail.T @ Vnew
    return out, S


def gdn_chunk_fwd(q, k, v, g, beta, S0=None, C: int = 64, scale: float = 1.0):
    """Scalar-decay GDN through the chunk form (D_t = alpha_t I, b = w = beta 1).

    q, k [B,T,Hk,Dk]; v [B,T,Hv,Dv]; g, beta [B,T,Hv]; S0 [B,Hv,Dk,Dv] or None.
    """
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    grp = Hv // Hk
    out = np.zeros((B, T, Hv, Dv))
    ST = np.zeros((B, Hv, Dk, Dv))
    for b in range(B):
        for hv in range(Hv):
            hk = hv // grp
            s0 = np.zeros((Dk, Dv)) if S0 is None else np.asarray(S0[b, hv], dtype=np.float64)
            gg = np.repeat(g[b, :, hv][:, None], Dk, axis=1)
            eb = np.repeat(beta[b, :, hv][:, None], Dk, axis=1)
            wb = np.repeat(beta[b, :, hv][:, None], Dv, axis=1)
            o, s = chunk_fwd_head(q[b, :, hk], k[b, :, hk], v[b, :, hv], gg, eb, wb, s0, C)
            out[b, :, hv] = scale * o
            ST[b, hv] = s
    return out, ST


def gdn2_chunk_fwd(q, k, v, g, eb, wb, S0=None, C: int = 64, scale: float = 1.0):
    """Gated DeltaNet-2 through the chunk form; g, eb [B,T,Hv,Dk], wb [B,T,Hv,Dv]."""
    q, k, v, g, eb, wb = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, eb, wb))
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    grp = Hv // Hk
    out = np.zeros((B, T, Hv, Dv))
    ST = np.zeros((B, Hv, Dk, Dv))
    for b in range(B):
        for hv in range(Hv):
            hk = hv // grp
            s0 = np.zeros((Dk, Dv)) if S0 is None else np.asarray(S0[b, hv], dtype=np.float64)
            o, s = chunk_fwd_head(q[b, :, hk], k[b, :, hk], v[b, :, hv], g[b, :, hv], eb[b, :, hv],
                                  wb[b, :, hv], s0, C)
            out[b, :, hv] = scale * o
            ST[b, hv] = s
    return out, ST
