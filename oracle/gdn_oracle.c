/*
 * gdn_oracle.c -- plain, slow, float64 CPU oracle of the Gated DeltaNet core.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load or run this code.  It shares nothing
 * with the GPU library: no headers, no helpers, no constants.
 *
 * Every input is widened exactly to double by the caller; every step below is
 * carried out in double, token by token, with no chunking, blocking or
 * reordering beyond what the formulas state.  Build flags: no fast-math and
 * -ffp-contract=off, so each multiply and add rounds as written.
 *
 * Sources (the pages this follows):
 *  - dingfen.github.io, "从 Full Attention 到 Gated DeltaNet", sections 9-10:
 *    the decay gate g = -exp(A_log) * softplus(a + dt_bias), alpha = exp(g),
 *    softplus(x) = log(1 + e^x), write strength beta = sigmoid(b), read-out
 *    y_t = S_t^T q_t.
 *  - rainlin-net.pages.dev "Qwen3.5", section "GDN详解": the gated delta rule
 *    S_t = alpha_t S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T with the
 *    read-out o_t = S_t q_t taken after the update.  The state is stored here
 *    as S[d_k][d_v], the transpose of that d_v x d_k matrix, so the rule reads
 *    S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T and the
 *    read-out o_t = S_t^T q_t.
 *  - zhichai.net "Gated DeltaNet-2", sections "Gated Delta Rule-2" and
 *    "退化兼容性": decoupled erase gate b_t (per key channel) and write gate
 *    w_t (per value channel), channel-wise decay D_t:
 *    S_t = (I - k_t e_t^T) D_t S_{t-1} + k_t z_t^T, e = b (.) k, z = w (.) v,
 *    expanded as Sbar = D S, r = Sbar^T e, S = Sbar + k (z - r)^T.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* softplus(x) = log(1 + e^x) (dingfen page, section 9), evaluated without
 * overflow: for x > 0, log(1 + e^x) = x + log(1 + e^-x). */
double oracle_softplus(double x) {
    if (x > 0.0) return x + log1p(exp(-x));
    return log1p(exp(x));
}

/* sigmoid(x) = 1 / (1 + e^-x) (dingfen page, section 10: beta = sigma(b)). */
double oracle_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Gate preparation for GDN (dingfen page sections 9-10; rainlin page module
 * code): for n token rows of Hv value heads,
 *   g[r,h]    = -exp(A_log[h]) * softplus(a[r,h] + dt_bias[h])   (log decay)
 *   beta[r,h] = sigmoid(b[r,h]).
 * One decay and one write strength per (token, value head). */
void oracle_gdn_gates(long n, int Hv, const double *a, const double *b,
                      const double *A_log, const double *dt_bias,
                      double *g, double *beta) {
    for (long r = 0; r < n; ++r)
        for (int h = 0; h < Hv; ++h) {
            long i = r * Hv + h;
            g[i] = -exp(A_log[h]) * oracle_softplus(a[i] + dt_bias[h]);
            beta[i] = oracle_sigmoid(b[i]);
        }
}

/* The gated delta rule, token by token (rainlin page, section "GDN详解").
 *   q, k : [B,T,Hk,Dk]   v, out : [B,T,Hv,Dv]   g, beta : [B,T,Hv]
 *   S0, ST : [B,Hv,Dk,Dv] (S0 may be NULL: zero initial state; ST may be NULL)
 * Value head hv reads key/query head hv / (Hv/Hk).  Each token applies the
 * transition P_t = alpha_t (I - beta_t k_t k_t^T) to the state and adds the
 * write beta_t k_t v_t^T.  P_t S is evaluated by distributing the product,
 *   P_t S = alpha_t S - alpha_t beta_t k_t (S^T k_t)^T,
 * which is the same matrix without forming the d_k x d_k factor; so
 *   S_t = alpha_t S_{t-1} + k_t (beta_t v_t - alpha_t beta_t S_{t-1}^T k_t)^T,
 * and o_t = scale * S_t^T q_t. */
void oracle_gdn_core(int B, int T, int Hk, int Hv, int Dk, int Dv,
                     const double *q, const double *k, const double *v,
                     const double *g, const double *beta, double scale,
                     const double *S0, double *out, double *ST) {
    const int grp = Hv / Hk;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < B * Hv; ++u) {
        const int bb = u / Hv, hv = u % Hv, hk = hv / grp;
        double *S = (double *)malloc(sizeof(double) * (size_t)Dk * Dv);
        double *sk = (double *)malloc(sizeof(double) * (size_t)Dv);  /* S_{t-1}^T k_t */
        double *w = (double *)malloc(sizeof(double) * (size_t)Dv);   /* column factor of the rank-one term */
        if (S0) memcpy(S, S0 + (size_t)u * Dk * Dv, sizeof(double) * (size_t)Dk * Dv);
        else memset(S, 0, sizeof(double) * (size_t)Dk * Dv);
        for (int t = 0; t < T; ++t) {
            const double *qt = q + (((size_t)bb * T + t) * Hk + hk) * Dk;
            const double *kt = k + (((size_t)bb * T + t) * Hk + hk) * Dk;
            const double *vt = v + (((size_t)bb * T + t) * Hv + hv) * Dv;
            const size_t gi = ((size_t)bb * T + t) * Hv + hv;
            const double alpha = exp(g[gi]);
            const double be = beta[gi];
            for (int j = 0; j < Dv; ++j) sk[j] = 0.0;
            for (int i = 0; i < Dk; ++i)
                for (int j = 0; j < Dv; ++j) sk[j] += S[(size_t)i * Dv + j] * kt[i];
            for (int j = 0; j < Dv; ++j) w[j] = be * vt[j] - alpha * be * sk[j];
            for (int i = 0; i < Dk; ++i)
                for (int j = 0; j < Dv; ++j)
                    S[(size_t)i * Dv + j] = alpha * S[(size_t)i * Dv + j] + kt[i] * w[j];
            double *ot = out + (((size_t)bb * T + t) * Hv + hv) * Dv;
            for (int j = 0; j < Dv; ++j) ot[j] = 0.0;
            for (int i = 0; i < Dk; ++i)
                for (int j = 0; j < Dv; ++j) ot[j] += S[(size_t)i * Dv + j] * qt[i];
            for (int j = 0; j < Dv; ++j) ot[j] *= scale;
        }
        if (ST) memcpy(ST + (size_t)u * Dk * Dv, S, sizeof(double) * (size_t)Dk * Dv);
        free(S);
        free(sk);
        free(w);
    }
}

/* GDN forward from raw gate logits: oracle_gdn_gates followed by
 * oracle_gdn_core.  a, b : [B,T,Hv]; A_log, dt_bias : [Hv]. */
void oracle_gdn_fwd(int B, int T, int Hk, int Hv, int Dk, int Dv,
                    const double *q, const double *k, const double *v,
                    const double *a, const double *b, const double *A_log,
                    const double *dt_bias, double scale, const double *S0,
                    double *out, double *ST) {
    const size_t n = (size_t)B * T * Hv;
    double *g = (double *)malloc(sizeof(double) * (n ? n : 1));
    double *beta = (double *)malloc(sizeof(double) * (n ? n : 1));
    oracle_gdn_gates((long)B * T, Hv, a, b, A_log, dt_bias, g, beta);
    oracle_gdn_core(B, T, Hk, Hv, Dk, Dv, q, k, v, g, beta, scale, S0, out, ST);
    free(g);
    free(beta);
}

/* Gate preparation for Gated DeltaNet-2.  The zhichai page fixes only that the
 * decay is channel-wise and that the erase gate lies in [0,1]^{d_k} and the
 * write gate in [0,1]^{d_v}; the forms below are this oracle's reading: the GDN
 * decay parametrisation per key channel (without dt_bias) and sigmoids of
 * raw logits.  Per (token row r, value head h, key channel c)
 *   g[r,h,c]  = -exp(A_log[h,c]) * softplus(a[r,h,c])   (channel-wise log decay)
 *   eb[r,h,c] = sigmoid(erase[r,h,c])                     (erase gate b_t)
 * and per value channel j: wb[r,h,j] = sigmoid(write[r,h,j]) (write gate w_t). */
void oracle_gdn2_gates(long n, int Hv, int Dk, int Dv, const double *a,
                       const double *A_log, const double *erase,
                       const double *write, double *g, double *eb, double *wb) {
    for (long r = 0; r < n; ++r)
        for (int h = 0; h < Hv; ++h) {
            for (int c = 0; c < Dk; ++c) {
                size_t i = ((size_t)r * Hv + h) * Dk + c;
                g[i] = -exp(A_log[(size_t)h * Dk + c]) * oracle_softplus(a[i]);
                eb[i] = oracle_sigmoid(erase[i]);
            }
            for (int j = 0; j < Dv; ++j) {
                size_t i = ((size_t)r * Hv + h) * Dv + j;
                wb[i] = oracle_sigmoid(write[i]);
            }
        }
}

/* Gated Delta Rule-2, token by token (zhichai page, expanded form):
 *   D = exp(g) (per key channel);  Sbar = diag(D) S;  e = eb (.) k;
 *   z = wb (.) v;  r = Sbar^T e;  S = Sbar + k (z - r)^T;  out = scale S^T q.
 *   g, eb : [B,T,Hv,Dk]   wb : [B,T,Hv,Dv]; other layouts as oracle_gdn_core. */
void oracle_gdn2_core(int B, int T, int Hk, int Hv, int Dk, int Dv,
                      const double *q, const double *k, const double *v,
                      const double *g, const double *eb, const double *wb,
                      double scale, const double *S0, double *out, double *ST) {
    const int grp = Hv / Hk;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < B * Hv; ++u) {
        const int bb = u / Hv, hv = u % Hv, hk = hv / grp;
        double *S = (double *)malloc(sizeof(double) * (size_t)Dk * Dv);
        double *e = (double *)malloc(sizeof(double) * (size_t)Dk);
        double *r = (double *)malloc(sizeof(double) * (size_t)Dv);
        if (S0) memcpy(S, S0 + (size_t)u * Dk * Dv, sizeof(double) * (size_t)Dk * Dv);
        else memset(S, 0, sizeof(double) * (size_t)Dk * Dv);
        for (int t = 0; t < T; ++t) {
            const double *qt = q + (((size_t)bb * T + t) * Hk + hk) * Dk;
            const double *kt = k + (((size_t)bb * T + t) * Hk + hk) * Dk;
            const double *vt = v + (((size_t)bb * T + t) * Hv + hv) * Dv;
            const size_t ci = (((size_t)bb * T + t) * Hv + hv) * Dk;
            const size_t vi = (((size_t)bb * T + t) * Hv + hv) * Dv;
            /* Sbar = diag(D) S: row i of S (key channel i) decays by exp(g_i) */
            for (int i = 0; i < Dk; ++i) {
                const double Di = exp(g[ci + i]);
                for (int j = 0; j < Dv; ++j) S[(size_t)i * Dv + j] *= Di;
            }
            /* e = erase gate (.) k */
            for (int i = 0; i < Dk; ++i) e[i] = eb[ci + i] * kt[i];
            /* r = Sbar^T e */
            for (int j = 0; j < Dv; ++j) r[j] = 0.0;
            for (int i = 0; i < Dk; ++i)
                for (int j = 0; j < Dv; ++j) r[j] += S[(size_t)i * Dv + j] * e[i];
            /* S = Sbar + k (z - r)^T with z = write gate (.) v */
            for (int j = 0; j < Dv; ++j) r[j] = wb[vi + j] * vt[j] - r[j];
            for (int i = 0; i < Dk; ++i)
                for (int j = 0; j < Dv; ++j) S[(size_t)i * Dv + j] += kt[i] * r[j];
            /* read-out after the update */
            double *ot = out + (((size_t)bb * T + t) * Hv + hv) * Dv;
            for (int j = 0; j < Dv; ++j) ot[j] = 0.0;
            for (int i = 0; i < Dk; ++i)
                for (int j = 0; j < Dv; ++j) ot[j] += S[(size_t)i * Dv + j] * qt[i];
            for (int j = 0; j < Dv; ++j) ot[j] *= scale;
        }
        if (ST) memcpy(ST + (size_t)u * Dk * Dv, S, sizeof(double) * (size_t)Dk * Dv);
        free(S);
        free(e);
        free(r);
    }
}

/* Gated DeltaNet-2 forward from raw logits: oracle_gdn2_gates + core.
 * a, erase : [B,T,Hv,Dk]; write : [B,T,Hv,Dv]; A_log : [Hv,Dk]. */
void oracle_gdn2_fwd(int B, int T, int Hk, int Hv, int Dk, int Dv,
                     const double *q, const double *k, const double *v,
                     const double *a, const double *A_log, const double *erase,
                     const double *write, double scale, const double *S0,
                     double *out, double *ST) {
    const size_t nk = (size_t)B * T * Hv * Dk, nv = (size_t)B * T * Hv * Dv;
    double *g = (double *)malloc(sizeof(double) * (nk ? nk : 1));
    double *eb = (double *)malloc(sizeof(double) * (nk ? nk : 1));
    double *wb = (double *)malloc(sizeof(double) * (nv ? nv : 1));
    oracle_gdn2_gates((long)B * T, Hv, Dk, Dv, a, A_log, erase, write, g, eb, wb);
    oracle_gdn2_core(B, T, Hk, Hv, Dk, Dv, q, k, v, g, eb, wb, scale, S0, out, ST);
    free(g);
    free(eb);
    free(wb);
}

/* Gated RMS normalisation of the core's output (rainlin-net.pages.dev
 * "Qwen3.5", section "GDN详解": the module passes the read-out through a gated
 * RMSNorm with the output gate z before the output projection; wanger-sjtu
 * page, section "输出门控与 RMSNorm": the gate works like SwiGLU's; 10100.com
 * pseudocode: a sigmoid output gate multiplied elementwise).  The pages give
 * no formula; the reading taken here: per row (one token of one value head,
 * d values)
 *     y_c = x_c / sqrt(mean_c(x_c^2) + eps) * w_c * act(z_c)
 * with act = SiLU (gate 0: z * sigmoid(z), the SwiGLU gate) or sigmoid
 * (gate 1).  rows x d row-major in x, z, y; w has d entries. */
void oracle_gated_rmsnorm(long rows, int d, const double *x, const double *z, const double *w,
                          double eps, int gate, double *y) {
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r) {
        const double *xr = x + r * d, *zr = z + r * d;
        double ss = 0.0;
        for (int c = 0; c < d; ++c) ss += xr[c] * xr[c];
        const double inv = 1.0 / sqrt(ss / d + eps);
        for (int c = 0; c < d; ++c) {
            const double s = oracle_sigmoid(zr[c]);
            const double act = gate == 0 ? zr[c] * s : s;
            y[r * d + c] = xr[c] * inv * w[c] * act;
        }
    }
}

/* Depthwise causal convolution over time with an optional SiLU, the prologue
 * that turns the mixed q|k|v projection into q, k, v (dingfen.github.io,
 * section 10: x -> Linear -> CausalConv1D -> SiLU -> (q, k, v); 10100.com:
 * kernel size 4; wanger-sjtu page: a depthwise causal conv over the mixed QKV
 * channels, with the conv inputs cached for decode).  Per sequence b, channel
 * c and token t (inputs before token 0 come from the cached state, or are 0):
 *     y[b,t,c] = act(bias[c] + sum_{j<K} w[c][j] x[b, t-K+1+j, c])
 * x, y [B][T][C]; w [C][K]; bias [C] or NULL; state [B][K-1][C] (the K-1
 * inputs before token 0, oldest first) or NULL; state_out [B][K-1][C] (the
 * last K-1 inputs, including older state when T < K-1) or NULL.
 * silu: act(x) = x sigmoid(x), else the identity. */
void oracle_causal_conv1d(int B, int T, int C, int K, const double *x, const double *w,
                          const double *bias, const double *state, int silu, double *y,
                          double *state_out) {
#pragma omp parallel for schedule(static)
    for (int b = 0; b < B; ++b) {
        for (int c = 0; c < C; ++c) {
            for (int t = 0; t < T; ++t) {
                double acc = bias ? bias[c] : 0.0;
                for (int j = 0; j < K; ++j) {
                    const int s = t - K + 1 + j;  /* input token; s < 0 reads the state */
                    double xv = 0.0;
                    if (s >= 0) xv = x[((size_t)b * T + s) * C + c];
                    else if (state) xv = state[((size_t)b * (K - 1) + (K - 1 + s)) * C + c];
                    acc += w[(size_t)c * K + j] * xv;
                }
                y[((size_t)b * T + t) * C + c] = silu ? acc * oracle_sigmoid(acc) : acc;
            }
            if (state_out) {
                for (int i = 0; i < K - 1; ++i) {
                    const int s = T - (K - 1) + i;  /* token of state slot i */
                    double xv = 0.0;
                    if (s >= 0) xv = x[((size_t)b * T + s) * C + c];
                    else if (state) xv = state[((size_t)b * (K - 1) + (K - 1 + s)) * C + c];
                    state_out[((size_t)b * (K - 1) + i) * C + c] = xv;
                }
            }
        }
    }
}

/* One Gated Delta Rule-2 token step on a d_k x d_v state (zhichai page, the
 * expanded form): S = diag(D) S;  r = S^T e;  S += k (z - r)^T.  r is scratch
 * of d_v entries. */
static void g2_step(int Dk, int Dv, double *S, const double *D, const double *e,
                    const double *k, const double *z, double *r) {
    for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j) S[(size_t)i * Dv + j] *= D[i];
    for (int j = 0; j < Dv; ++j) r[j] = 0.0;
    for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j) r[j] += S[(size_t)i * Dv + j] * e[i];
    for (int j = 0; j < Dv; ++j) r[j] = z[j] - r[j];
    for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j) S[(size_t)i * Dv + j] += k[i] * r[j];
}

/* Gradient of the Gated DeltaNet-2 forward (oracle_gdn2_fwd) by reverse-mode
 * differentiation of the token loop (zhichai page, sections "Gated Delta
 * Rule-2" for the recurrence and "Gate-aware 反向传播" for the requirement that
 * the gate factors stay at each token instead of being pulled out of the
 * accumulation).  The scalar being differentiated is
 *     L = sum(d_out * out) + sum(d_ST * S_T),
 * so the results are the vector-Jacobian products of the forward with the
 * given output and final-state gradients (d_ST NULL = 0).
 *
 * Per token, with D = exp(g), e = eb (.) k, z = wb (.) v, the forward step is
 * Sbar = diag(D) S_prev, r = Sbar^T e, S = Sbar + k (z - r)^T, o = scale S^T q;
 * its adjoint, given dS (the gradient of S after the step), is
 *     dS += scale q do^T;          dq = scale S do
 *     dk += dS (z - r);            dz = dS^T k;        dr = -dz
 *     dSbar = dS + e dr^T;         de = Sbar dr
 *     dD_i = sum_j dSbar_ij S_prev_ij;   dS_prev = diag(D) dSbar
 * and through the gates g = -exp(A_log) softplus(a), eb = sigmoid(erase),
 * wb = sigmoid(write):
 *     dg = dD D;  da = -dg exp(A_log) sigmoid(a);  dA_log += dg g
 *     dk += de eb;  d_erase = de k eb (1 - eb);  dv = dz wb;
 *     d_write = dz v wb (1 - wb).
 * The states before each token are needed in reverse order; they are kept
 * every SEG tokens and recomputed inside each stretch of SEG tokens with the
 * same forward step, which reproduces them exactly.
 * Layouts: dq, dk [B,T,Hk,Dk] (summed over the value heads of a key head);
 * dv, d_write [B,T,Hv,Dv]; da, d_erase [B,T,Hv,Dk]; dA_log [Hv,Dk]; dS0
 * [B,Hv,Dk,Dv] (the gradient of the initial state, S0 NULL = 0). */
#define G2_SEG 64
void oracle_gdn2_bwd(int B, int T, int Hk, int Hv, int Dk, int Dv,
                     const double *q, const double *k, const double *v,
                     const double *a, const double *A_log, const double *erase,
                     const double *write, double scale, const double *S0,
                     const double *dout, const double *dST, double *dq, double *dk,
                     double *dv, double *da, double *derase, double *dwrite,
                     double *dA_log, double *dS0) {
    const int grp = Hv / Hk;
    const size_t nk = (size_t)B * T * Hv * Dk, nv = (size_t)B * T * Hv * Dv, SS = (size_t)Dk * Dv;
    double *g = (double *)malloc(sizeof(double) * (nk ? nk : 1));
    double *eb = (double *)malloc(sizeof(double) * (nk ? nk : 1));
    double *wb = (double *)malloc(sizeof(double) * (nv ? nv : 1));
    /* per value head gradients of q and k, summed over each key head's group below */
    double *dqh = (double *)calloc(nk ? nk : 1, sizeof(double));
    double *dkh = (double *)calloc(nk ? nk : 1, sizeof(double));
    double *dal = (double *)calloc((size_t)B * Hv * Dk, sizeof(double));
    oracle_gdn2_gates((long)B * T, Hv, Dk, Dv, a, A_log, erase, write, g, eb, wb);
    const int nseg = (T + G2_SEG - 1) / G2_SEG;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < B * Hv; ++u) {
        const int bb = u / Hv, hv = u % Hv, hk = hv / grp;
        double *cp = (double *)malloc(sizeof(double) * SS * (nseg ? nseg : 1));
        double *st = (double *)malloc(sizeof(double) * SS * G2_SEG);
        double *S = (double *)malloc(sizeof(double) * SS);
        double *Sb = (double *)malloc(sizeof(double) * SS);
        double *dS = (double *)malloc(sizeof(double) * SS);
        double *D = (double *)malloc(sizeof(double) * Dk);
        double *e = (double *)malloc(sizeof(double) * Dk);
        double *de = (double *)malloc(sizeof(double) * Dk);
        double *z = (double *)malloc(sizeof(double) * Dv);
        double *dl = (double *)malloc(sizeof(double) * Dv);
        double *dz = (double *)malloc(sizeof(double) * Dv);
        double *r = (double *)malloc(sizeof(double) * Dv);
#define TOK_GATES(t)                                                                  \
        const size_t ci = (((size_t)bb * T + (t)) * Hv + hv) * Dk;                    \
        const size_t vi = (((size_t)bb * T + (t)) * Hv + hv) * Dv;                    \
        const double *kt = k + (((size_t)bb * T + (t)) * Hk + hk) * Dk;               \
        const double *vt = v + vi;                                                    \
        for (int i = 0; i < Dk; ++i) { D[i] = exp(g[ci + i]); e[i] = eb[ci + i] * kt[i]; } \
        for (int j = 0; j < Dv; ++j) z[j] = wb[vi + j] * vt[j];
        /* forward pass keeping the state before every SEG-th token */
        if (S0) memcpy(S, S0 + (size_t)u * SS, sizeof(double) * SS);
        else memset(S, 0, sizeof(double) * SS);
        for (int t = 0; t < T; ++t) {
            if (t % G2_SEG == 0) memcpy(cp + (size_t)(t / G2_SEG) * SS, S, sizeof(double) * SS);
            TOK_GATES(t)
            g2_step(Dk, Dv, S, D, e, kt, z, r);
        }
        if (dST) memcpy(dS, dST + (size_t)u * SS, sizeof(double) * SS);
        else memset(dS, 0, sizeof(double) * SS);
        for (int s = nseg - 1; s >= 0; --s) {
            const int t0 = s * G2_SEG, len = (T - t0 < G2_SEG) ? T - t0 : G2_SEG;
            /* st[j] = state before token t0 + j */
            memcpy(S, cp + (size_t)s * SS, sizeof(double) * SS);
            for (int j = 0; j < len; ++j) {
                memcpy(st + (size_t)j * SS, S, sizeof(double) * SS);
                if (j + 1 < len) {
                    TOK_GATES(t0 + j)
                    g2_step(Dk, Dv, S, D, e, kt, z, r);
                }
            }
            for (int j = len - 1; j >= 0; --j) {
                const int t = t0 + j;
                TOK_GATES(t)
                const double *Sp = st + (size_t)j * SS;
                const double *qt = q + (((size_t)bb * T + t) * Hk + hk) * Dk;
                const double *dot = dout + vi;
                /* recompute Sbar, r, delta = z - r and S after the step */
                for (int i = 0; i < Dk; ++i)
                    for (int jj = 0; jj < Dv; ++jj) Sb[(size_t)i * Dv + jj] = Sp[(size_t)i * Dv + jj] * D[i];
                for (int jj = 0; jj < Dv; ++jj) r[jj] = 0.0;
                for (int i = 0; i < Dk; ++i)
                    for (int jj = 0; jj < Dv; ++jj) r[jj] += Sb[(size_t)i * Dv + jj] * e[i];
                for (int jj = 0; jj < Dv; ++jj) dl[jj] = z[jj] - r[jj];
                for (int i = 0; i < Dk; ++i)
                    for (int jj = 0; jj < Dv; ++jj)
                        S[(size_t)i * Dv + jj] = Sb[(size_t)i * Dv + jj] + kt[i] * dl[jj];
                /* read-out: o = scale S^T q */
                double *dqt = dqh + ci, *dkt = dkh + ci;
                for (int i = 0; i < Dk; ++i) {
                    double acc = 0.0;
                    for (int jj = 0; jj < Dv; ++jj) acc += S[(size_t)i * Dv + jj] * dot[jj];
                    dqt[i] += scale * acc;
                }
                for (int i = 0; i < Dk; ++i)
                    for (int jj = 0; jj < Dv; ++jj) dS[(size_t)i * Dv + jj] += scale * qt[i] * dot[jj];
                /* S = Sbar + k delta^T */
                for (int i = 0; i < Dk; ++i) {
                    double acc = 0.0;
                    for (int jj = 0; jj < Dv; ++jj) acc += dS[(size_t)i * Dv + jj] * dl[jj];
                    dkt[i] += acc;
                }
                for (int jj = 0; jj < Dv; ++jj) dz[jj] = 0.0;
                for (int i = 0; i < Dk; ++i)
                    for (int jj = 0; jj < Dv; ++jj) dz[jj] += dS[(size_t)i * Dv + jj] * kt[i];
                /* r = Sbar^T e, dr = -dz: dSbar = dS - e dz^T, de = -Sbar dz */
                for (int i = 0; i < Dk; ++i) {
                    double acc = 0.0;
                    for (int jj = 0; jj < Dv; ++jj) acc += Sb[(size_t)i * Dv + jj] * dz[jj];
                    de[i] = -acc;
                }
                for (int i = 0; i < Dk; ++i)
                    for (int jj = 0; jj < Dv; ++jj) dS[(size_t)i * Dv + jj] -= e[i] * dz[jj];
                /* Sbar = diag(D) S_prev */
                for (int i = 0; i < Dk; ++i) {
                    double dD = 0.0;
                    for (int jj = 0; jj < Dv; ++jj) dD += dS[(size_t)i * Dv + jj] * Sp[(size_t)i * Dv + jj];
                    for (int jj = 0; jj < Dv; ++jj) dS[(size_t)i * Dv + jj] *= D[i];
                    const double dg = dD * D[i];
                    const double Ai = A_log[(size_t)hv * Dk + i];
                    da[ci + i] = -dg * exp(Ai) * oracle_sigmoid(a[ci + i]);
                    dal[(size_t)u * Dk + i] += dg * g[ci + i];
                    /* e = eb (.) k */
                    dkt[i] += de[i] * eb[ci + i];
                    derase[ci + i] = de[i] * kt[i] * eb[ci + i] * (1.0 - eb[ci + i]);
                }
                /* z = wb (.) v */
                for (int jj = 0; jj < Dv; ++jj) {
                    dv[vi + jj] = dz[jj] * wb[vi + jj];
                    dwrite[vi + jj] = dz[jj] * vt[jj] * wb[vi + jj] * (1.0 - wb[vi + jj]);
                }
            }
        }
#undef TOK_GATES
        memcpy(dS0 + (size_t)u * SS, dS, sizeof(double) * SS);
        free(cp); free(st); free(S); free(Sb); free(dS);
        free(D); free(e); free(de); free(z); free(dl); free(dz); free(r);
    }
    /* sums over the value heads of each key head, and over sequences for A_log */
    for (int bb = 0; bb < B; ++bb)
        for (int t = 0; t < T; ++t)
            for (int hk = 0; hk < Hk; ++hk)
                for (int i = 0; i < Dk; ++i) {
                    double sq = 0.0, sk = 0.0;
                    for (int x = 0; x < grp; ++x) {
                        const size_t ci = (((size_t)bb * T + t) * Hv + hk * grp + x) * Dk + i;
                        sq += dqh[ci];
                        sk += dkh[ci];
                    }
                    dq[(((size_t)bb * T + t) * Hk + hk) * Dk + i] = sq;
                    dk[(((size_t)bb * T + t) * Hk + hk) * Dk + i] = sk;
                }
    for (int hv = 0; hv < Hv; ++hv)
        for (int i = 0; i < Dk; ++i) {
            double s = 0.0;
            for (int bb = 0; bb < B; ++bb) s += dal[((size_t)bb * Hv + hv) * Dk + i];
            dA_log[(size_t)hv * Dk + i] = s;
        }
    free(g); free(eb); free(wb); free(dqh); free(dkh); free(dal);
}
