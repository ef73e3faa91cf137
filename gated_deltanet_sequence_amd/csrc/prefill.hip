// prefill.hip -- chunkwise-parallel prefill of the gated delta rule.
//
// Method: the WY chunk form of zhichai.net's "Gated DeltaNet-2" digest
// (section "高效训练：WY 算法依然成立") in its scalar-decay case (same page,
// section "退化兼容性": D_t = alpha_t I and both gates equal beta_t), with the
// state stored as S[d_k][d_v].  Inside a chunk of C = 64 tokens with in-chunk
// cumulative log decay G_r (gamma_r = e^{G_r}) and chunk-start state S:
//
//   L     = strictly-lower( beta_r e^{G_r - G_i} k_r.k_i )          (C x C)
//   A     = (I + L)^{-1}
//   Delta = A (beta (.) V - beta gamma (.) K S)     (= U - W S of the page)
//   O     = gamma (.) (Q S) + A_qk Delta,  A_qk = lower-incl-diag(e^{G_r-G_i} q_r.k_i)
//   S'    = gamma_C S + K^T (eta (.) Delta),  eta_i = e^{G_C - G_i}
//
// Delta is formed as A times the residual instead of U - W S (W = A diag(beta
// gamma) K, U = A diag(beta) V): the same numbers, one C x C x d_k product fewer.
// Every decay factor is a difference of cumulative logs (all <= 1), never a
// 1/gamma, so nothing overflows however strong the decay.
//
// Three kernels (the hot path):
//  1. gate_prep   -- g = -exp(A_log) softplus(a + dt_bias) and beta = sigmoid(b)
//                    per token (float32), and the in-chunk inclusive prefix sum
//                    G of g (float64, so that e^{G_r - G_i} keeps float32
//                    accuracy when |G| is in the hundreds).
//  2. chunk_local -- per (sequence, key head, chunk): K K^T and Q K^T on the
//                    matrix cores (shared by the Hv/Hk value heads of the key
//                    head), then per value head the gating, the LDS-resident
//                    blocked inverse of (I + L) and the operand fragments of A
//                    and A_qk for the scan.  Fully parallel over chunks.
//  3. state_scan  -- per (sequence, value head, 64 state columns): the float32
//                    state lives in matrix-core accumulators (4 waves x 16
//                    columns); the kernel walks the chunks in order and does the
//                    five dense products per chunk on the matrix cores.
//
// Operand type of the products: float16 for bfloat16 inputs (11-bit
// significand; bf16 operands would exceed the 2e-3 error budget), float32 for
// float32 inputs.  Accumulation is float32 throughout.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

static constexpr int C = 64;       // chunk length
static constexpr int NPAIR = 6;    // operand fragments of a strictly-lower 64x64 matrix

// Pair fragments of a strictly-lower 64x64 matrix: row tile r (16 rows) needs
// k-steps q = 0..r/2 (32 columns each); pair_index numbers them 0..5.
__host__ __device__ constexpr int pair_base(int r) { return r == 0 ? 0 : r == 1 ? 1 : r == 2 ? 2 : 4; }
__host__ __device__ constexpr int pair_index(int r, int q) { return pair_base(r) + q; }

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t prefill_workspace_layout(int B, int T, int Hv, bool f32, void *base, PrefillWorkspace *ws) {
    const size_t NC = (size_t)(T + C - 1) / C;
    const size_t units = (size_t)B * Hv * NC;
    const size_t esz = f32 ? 4 : 2;
    size_t off = 0;
    const size_t oG = off;    off = align256(off + units * C * sizeof(double));
    const size_t oB = off;    off = align256(off + units * C * sizeof(float));
    const size_t oT = off;    off = align256(off + units * C * 4 * sizeof(float));
    const size_t oA = off;    off = align256(off + units * NPAIR * 64 * 8 * esz);
    const size_t oQ = off;    off = align256(off + units * NPAIR * 64 * 8 * esz);
    if (ws) {
        char *p = (char *)base;
        ws->G = (double *)(p + oG);
        ws->beta = (float *)(p + oB);
        ws->tok = (float *)(p + oT);
        ws->apair = p + oA;
        ws->qpair = p + oQ;
        ws->bytes = off;
    }
    return off;
}

// ---------------------------------------------------------------------------
// 1. gate preparation: one wave per (sequence, value head, chunk), lane = token
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gate_prep_kernel(int B, int T, int Hv, int NC,
                                                        const float *__restrict__ a,
                                                        const float *__restrict__ b,
                                                        const float *__restrict__ A_log,
                                                        const float *__restrict__ dt_bias,
                                                        double *__restrict__ Gout,
                                                        float *__restrict__ beta_out) {
    const int lane = threadIdx.x & 63;
    const long unit = (long)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b*Hv + hv)*NC + n
    if (unit >= (long)B * Hv * NC) return;
    const int n = (int)(unit % NC);
    const long bh = unit / NC;
    const int hv = (int)(bh % Hv);
    const int bb = (int)(bh / Hv);
    const int t = n * C + lane;
    float g = 0.f, be = 0.f;
    if (t < T) {
        const size_t i = ((size_t)bb * T + t) * Hv + hv;
        g = -expf(A_log[hv]) * softplus_f32(a[i] + dt_bias[hv]);
        be = sigmoid_f32(b[i]);
    }
    double G = (double)g;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(G, off, 64);
        if (lane >= off) G += y;
    }
    Gout[unit * C + lane] = G;
    beta_out[unit * C + lane] = be;
}

// ---------------------------------------------------------------------------
// Shared helpers for the matrix-core products.
// X is a row-major LDS matrix with row stride `ld` elements.  The k-block
// operand of row `row`, contraction block starting at column k0 is the 4
// consecutive values X[row][k0 + 4*(lane/16) + i].
// ---------------------------------------------------------------------------
template <bool F32>
__device__ __forceinline__ typename mma<F32>::V4 lds_kblock(const typename mma<F32>::E *X,
                                                            int ld, int row, int k0, int g) {
    return *reinterpret_cast<const typename mma<F32>::V4 *>(X + (size_t)row * ld + k0 + 4 * g);
}

// Off-diagonal blocks of column block JB of X = (I + L)^{-1} (16x16 blocks,
// diagonal blocks already in Xm):  X[i][JB] = -X[i][i] sum_{mb=JB}^{i-1} L[i][mb] X[mb][JB].
// The column's blocks stay in accumulator layout, which is the B-operand layout
// of the next product; float32 matrix-core products.
template <int JB, int LDF>
__device__ __forceinline__ void inverse_column(const float *Lm, float *Xm, int m, int g) {
    f4 Xcol[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) Xcol[JB][s] = Xm[(16 * JB + 4 * g + s) * LDF + 16 * JB + m];
#pragma unroll
    for (int ib = JB + 1; ib < 4; ++ib) {
        f4 Tacc = {0, 0, 0, 0};
#pragma unroll
        for (int mb = JB; mb < ib; ++mb) {
            const f4 av = *reinterpret_cast<const f4 *>(Lm + (16 * ib + m) * LDF + 16 * mb + 4 * g);
            Tacc = mma<true>::block(Tacc, av, Xcol[mb]);
        }
        const f4 dv = *reinterpret_cast<const f4 *>(Xm + (16 * ib + m) * LDF + 16 * ib + 4 * g);
        f4 Xn = {0, 0, 0, 0};
        Xn = -mma<true>::block(Xn, dv, Tacc);
        Xcol[ib] = Xn;
#pragma unroll
        for (int s = 0; s < 4; ++s) Xm[(16 * ib + 4 * g + s) * LDF + 16 * JB + m] = Xn[s];
    }
}

// ---------------------------------------------------------------------------
// 2. chunk-local WY auxiliaries
// ---------------------------------------------------------------------------
template <bool F32, typename TIn, int DK>
struct ChunkLocalSmem {
    typedef typename mma<F32>::E E;
    static constexpr int LDX = DK + (F32 ? 4 : 8);   // row stride of Q/K staging (elements)
    static constexpr int LDF = C + 4;                // row stride of float32 64x64 matrices
    static constexpr size_t QK_BYTES = (size_t)2 * C * LDX * sizeof(E);
    static constexpr size_t LX_BYTES = (size_t)2 * C * LDF * sizeof(float);
    static constexpr size_t U_BYTES = QK_BYTES > LX_BYTES ? QK_BYTES : LX_BYTES;
};

template <bool F32, typename TIn, int DK>
__global__ __launch_bounds__(256) void chunk_local_kernel(
    int B, int T, int Hk, int Hv, int NC, const TIn *__restrict__ q, const TIn *__restrict__ k,
    const double *__restrict__ Gin, const float *__restrict__ beta_in, float *__restrict__ tok,
    typename mma<F32>::E *__restrict__ apair, typename mma<F32>::E *__restrict__ qpair) {
    typedef ChunkLocalSmem<F32, TIn, DK> SM;
    typedef typename mma<F32>::E E;
    typedef typename mma<F32>::V4 V4;
    constexpr int LDX = SM::LDX, LDF = SM::LDF;

    // union: Q/K staging (phase 1) | gated L and the inverse X (phase 2)
    __shared__ __attribute__((aligned(16))) char u_raw[SM::U_BYTES];
    __shared__ __attribute__((aligned(16))) float KK[C * LDF];
    __shared__ __attribute__((aligned(16))) float QK[C * LDF];
    __shared__ double Gs[C];
    __shared__ float Bs[C];
    E *Xq = reinterpret_cast<E *>(u_raw);
    E *Xk = Xq + C * LDX;
    float *Lm = reinterpret_cast<float *>(u_raw);
    float *Xm = Lm + C * LDF;

    const int n = blockIdx.x, hk = blockIdx.y, bb = blockIdx.z;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, m = lane & 15;
    const int G = Hv / Hk;
    const int t0 = n * C;

    // ---- stage Q and K rows of this chunk (zero past the end)
    for (int idx = tid; idx < C * (DK / 8); idx += 256) {
        const int r = idx / (DK / 8), c8 = (idx % (DK / 8)) * 8;
        f4 q0 = {0, 0, 0, 0}, q1 = q0, k0 = q0, k1 = q0;
        if (t0 + r < T) {
            const size_t off = (((size_t)bb * T + t0 + r) * Hk + hk) * DK + c8;
            ld8(q, off, q0, q1);
            ld8(k, off, k0, k1);
        }
        *reinterpret_cast<V4 *>(Xq + r * LDX + c8) = mma<F32>::from_f4(q0);
        *reinterpret_cast<V4 *>(Xq + r * LDX + c8 + 4) = mma<F32>::from_f4(q1);
        *reinterpret_cast<V4 *>(Xk + r * LDX + c8) = mma<F32>::from_f4(k0);
        *reinterpret_cast<V4 *>(Xk + r * LDX + c8 + 4) = mma<F32>::from_f4(k1);
    }
    __syncthreads();

    // ---- K K^T and Q K^T, lower-triangular 16x16 tiles (10 each), 5 per wave
    for (int job = w; job < 20; job += 4) {
        const E *X = job < 10 ? Xk : Xq;
        float *Dst = job < 10 ? KK : QK;
        const int p = job % 10;
        const int rt = p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3;
        const int ct = p - (rt * (rt + 1)) / 2;
        f4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int kq = 0; kq < DK / 32; ++kq) {
            const V4 a0 = lds_kblock<F32>(X, LDX, 16 * rt + m, 32 * kq, g);
            const V4 a1 = lds_kblock<F32>(X, LDX, 16 * rt + m, 32 * kq + 16, g);
            const V4 b0 = lds_kblock<F32>(Xk, LDX, 16 * ct + m, 32 * kq, g);
            const V4 b1 = lds_kblock<F32>(Xk, LDX, 16 * ct + m, 32 * kq + 16, g);
            acc = mma<F32>::pair(acc, a0, a1, b0, b1);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) Dst[(16 * rt + 4 * g + i) * LDF + 16 * ct + m] = acc[i];
    }
    __syncthreads();  // Q/K staging is dead from here on: the union becomes L and X

    for (int j = 0; j < G; ++j) {
        const int hv = hk * G + j;
        const size_t unit = ((size_t)bb * Hv + hv) * NC + n;
        if (tid < C) {
            Gs[tid] = Gin[unit * C + tid];
            Bs[tid] = beta_in[unit * C + tid];
        }
        __syncthreads();

        // ---- L = strictly-lower(beta_r e^{G_r - G_i} KK[r][i]); zero elsewhere
        for (int e = tid; e < C * C; e += 256) {
            const int r = e / C, i = e % C;
            float val = 0.f;
            if (i < r) val = Bs[r] * expf((float)(Gs[r] - Gs[i])) * KK[r * LDF + i];
            Lm[r * LDF + i] = val;
        }
        __syncthreads();

        // ---- diagonal 16x16 blocks of X = (I + L)^{-1}: wave w, lane c < 16
        //      solves column c of block w by forward substitution in registers
        if (lane < 16) {
            const int o = 16 * w, c = lane;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s = (r == c) ? 1.f : 0.f;
#pragma unroll
                for (int jj = 0; jj < r; ++jj) s -= Lm[(o + r) * LDF + o + jj] * x[jj];
                x[r] = s;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) Xm[(o + r) * LDF + o + c] = x[r];
        }
        __syncthreads();

        // ---- off-diagonal blocks: wave w completes column block w
        if (w == 0) inverse_column<0, LDF>(Lm, Xm, m, g);
        else if (w == 1) inverse_column<1, LDF>(Lm, Xm, m, g);
        else if (w == 2) inverse_column<2, LDF>(Lm, Xm, m, g);
        __syncthreads();

        // ---- operand fragments for the scan: 6 pairs x 64 lanes per matrix.
        //      pair (r, q): lane (m, g) holds M[16r+m][32q + 4g + i] (i < 4) and
        //      M[16r+m][32q + 16 + 4g + i]; strictly-lower part only.
        E *ap = apair + unit * (NPAIR * 64 * 8);
        E *qp = qpair + unit * (NPAIR * 64 * 8);
        for (int job = tid; job < 2 * NPAIR * 64; job += 256) {
            const bool isA = job < NPAIR * 64;
            const int jj = job % (NPAIR * 64);
            const int p = jj / 64, l = jj % 64;
            const int r = p < 1 ? 0 : p < 2 ? 1 : p < 4 ? 2 : 3;
            const int qq = p - pair_base(r);
            const int row = 16 * r + (l & 15), gg = l >> 4;
            f4 v0, v1;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f4 vv;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int col = 32 * qq + 16 * h + 4 * gg + i;
                    float x = 0.f;
                    if (col < row) {
                        if (isA) x = Xm[row * LDF + col];
                        else x = expf((float)(Gs[row] - Gs[col])) * QK[row * LDF + col];
                    }
                    vv[i] = x;
                }
                if (h == 0) v0 = vv; else v1 = vv;
            }
            E *dst = (isA ? ap : qp) + (size_t)(p * 64 + l) * 8;
            *reinterpret_cast<V4 *>(dst) = mma<F32>::from_f4(v0);
            *reinterpret_cast<V4 *>(dst + 4) = mma<F32>::from_f4(v1);
        }
        if (tid < C) {
            const double Gl = Gs[C - 1];
            f4 rec;
            rec[0] = Bs[tid];
            rec[1] = expf((float)Gs[tid]);
            rec[2] = expf((float)(Gl - Gs[tid]));
            rec[3] = QK[tid * LDF + tid];
            *reinterpret_cast<f4 *>(tok + (unit * C + tid) * 4) = rec;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// 3. inter-chunk state scan with fused output
// ---------------------------------------------------------------------------
template <bool F32, int DK>
struct ScanSmem {
    typedef typename mma<F32>::E E;
    static constexpr int LDX = DK + (F32 ? 4 : 8);  // Q/K rows
    static constexpr int LDT = C + (F32 ? 4 : 8);   // K^T rows
};

template <bool F32, typename TIn, int DK, int DV>
__global__ __launch_bounds__(256) void state_scan_kernel(
    int B, int T, int Hk, int Hv, int NC, float scale, const TIn *__restrict__ q,
    const TIn *__restrict__ k, const TIn *__restrict__ v, const float *__restrict__ tok,
    const typename mma<F32>::E *__restrict__ apair, const typename mma<F32>::E *__restrict__ qpair,
    const float *__restrict__ S0, TIn *__restrict__ out, float *__restrict__ ST) {
    typedef ScanSmem<F32, DK> SM;
    typedef typename mma<F32>::E E;
    typedef typename mma<F32>::V4 V4;
    constexpr int LDX = SM::LDX, LDT = SM::LDT;
    constexpr int NKB = DK / 16;  // 16-row blocks of the state

    __shared__ __attribute__((aligned(16))) E Qs[C * LDX];
    __shared__ __attribute__((aligned(16))) E Ks[C * LDX];
    __shared__ __attribute__((aligned(16))) E Kt[DK * LDT];
    __shared__ __attribute__((aligned(16))) float Vt[C * 64];
    __shared__ __attribute__((aligned(16))) f4 Tk[C];

    constexpr int NCG = DV / 64;
    const int cg = blockIdx.x % NCG;
    const int hv = (blockIdx.x / NCG) % Hv;
    const int bb = blockIdx.x / (NCG * Hv);
    const int hk = hv / (Hv / Hk);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, m = lane & 15;
    const int col = 64 * cg + 16 * w + m;  // this lane's state column

    // state S[16kb + 4g + i][col] in accumulator tiles
    f4 S[NKB];
    {
        const size_t sb = ((size_t)bb * Hv + hv) * DK * DV;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[kb][i] = S0 ? S0[sb + (size_t)(16 * kb + 4 * g + i) * DV + col] : 0.f;
    }

    for (int n = 0; n < NC; ++n) {
        const int t0 = n * C;
        const size_t unit = ((size_t)bb * Hv + hv) * NC + n;
        __syncthreads();
        // ---- stage this chunk: Q, K rows (+ K^T), this group's 64 V columns, token records
        for (int idx = tid; idx < C * (DK / 8); idx += 256) {
            const int r = idx / (DK / 8), c8 = (idx % (DK / 8)) * 8;
            f4 q0 = {0, 0, 0, 0}, q1 = q0, k0 = q0, k1 = q0;
            if (t0 + r < T) {
                const size_t off = (((size_t)bb * T + t0 + r) * Hk + hk) * DK + c8;
                ld8(q, off, q0, q1);
                ld8(k, off, k0, k1);
            }
            *reinterpret_cast<V4 *>(Qs + r * LDX + c8) = mma<F32>::from_f4(q0);
            *reinterpret_cast<V4 *>(Qs + r * LDX + c8 + 4) = mma<F32>::from_f4(q1);
            const V4 kk0 = mma<F32>::from_f4(k0), kk1 = mma<F32>::from_f4(k1);
            *reinterpret_cast<V4 *>(Ks + r * LDX + c8) = kk0;
            *reinterpret_cast<V4 *>(Ks + r * LDX + c8 + 4) = kk1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Kt[(c8 + i) * LDT + r] = kk0[i];
                Kt[(c8 + 4 + i) * LDT + r] = kk1[i];
            }
        }
        for (int idx = tid; idx < C * 16; idx += 256) {
            const int r = idx / 16, c4 = (idx % 16) * 4;
            f4 vv = {0, 0, 0, 0};
            if (t0 + r < T) vv = ld4(v, (((size_t)bb * T + t0 + r) * Hv + hv) * DV + 64 * cg + c4);
            *reinterpret_cast<f4 *>(Vt + r * 64 + c4) = vv;
        }
        if (tid < C) Tk[tid] = *reinterpret_cast<const f4 *>(tok + (unit * C + tid) * 4);
        __syncthreads();

        // ---- B operands of the state
        V4 Sb[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) Sb[kb] = mma<F32>::from_f4(S[kb]);

        // ---- P = K S and Qa = Q S (64 x 16 per wave)
        f4 P[4], Qa[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            f4 pa = {0, 0, 0, 0}, qa = {0, 0, 0, 0};
#pragma unroll
            for (int kq = 0; kq < DK / 32; ++kq) {
                const V4 ka0 = lds_kblock<F32>(Ks, LDX, 16 * r + m, 32 * kq, g);
                const V4 ka1 = lds_kblock<F32>(Ks, LDX, 16 * r + m, 32 * kq + 16, g);
                pa = mma<F32>::pair(pa, ka0, ka1, Sb[2 * kq], Sb[2 * kq + 1]);
                const V4 qa0 = lds_kblock<F32>(Qs, LDX, 16 * r + m, 32 * kq, g);
                const V4 qa1 = lds_kblock<F32>(Qs, LDX, 16 * r + m, 32 * kq + 16, g);
                qa = mma<F32>::pair(qa, qa0, qa1, Sb[2 * kq], Sb[2 * kq + 1]);
            }
            P[r] = pa;
            Qa[r] = qa;
        }

        // ---- residual R = beta (.) V - beta gamma (.) P
        f4 R[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * r + 4 * g + i;
                const f4 tr = Tk[row];
                R[r][i] = tr[0] * (Vt[row * 64 + 16 * w + m] - tr[1] * P[r][i]);
            }
        V4 Rb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) Rb[r] = mma<F32>::from_f4(R[r]);

        // ---- Delta = R + strictly-lower(A) R
        const E *ap = apair + unit * (NPAIR * 64 * 8) + lane * 8;
        const E *qp = qpair + unit * (NPAIR * 64 * 8) + lane * 8;
        f4 D[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            f4 acc = R[r];
#pragma unroll
            for (int qq = 0; qq <= r / 2; ++qq) {
                const E *src = ap + (size_t)pair_index(r, qq) * 64 * 8;
                const V4 a0 = *reinterpret_cast<const V4 *>(src);
                const V4 a1 = *reinterpret_cast<const V4 *>(src + 4);
                acc = mma<F32>::pair(acc, a0, a1, Rb[2 * qq], Rb[2 * qq + 1]);
            }
            D[r] = acc;
        }
        V4 Db[4], De[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            Db[r] = mma<F32>::from_f4(D[r]);
            f4 de;
#pragma unroll
            for (int i = 0; i < 4; ++i) de[i] = Tk[16 * r + 4 * g + i][2] * D[r][i];
            De[r] = mma<F32>::from_f4(de);
        }

        // ---- O = gamma (.) Qa + diag(q.k) Delta + strictly-lower(A_qk) Delta
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            f4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f4 tr = Tk[16 * r + 4 * g + i];
                acc[i] = tr[1] * Qa[r][i] + tr[3] * D[r][i];
            }
#pragma unroll
            for (int qq = 0; qq <= r / 2; ++qq) {
                const E *src = qp + (size_t)pair_index(r, qq) * 64 * 8;
                const V4 a0 = *reinterpret_cast<const V4 *>(src);
                const V4 a1 = *reinterpret_cast<const V4 *>(src + 4);
                acc = mma<F32>::pair(acc, a0, a1, Db[2 * qq], Db[2 * qq + 1]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + 16 * r + 4 * g + i;
                if (t < T) io<TIn>::st(out, (((size_t)bb * T + t) * Hv + hv) * DV + col, scale * acc[i]);
            }
        }

        // ---- S = gamma_C S + K^T (eta (.) Delta)
        const float gC = Tk[C - 1][1];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            f4 acc = gC * S[kb];
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
                const V4 a0 = lds_kblock<F32>(Kt, LDT, 16 * kb + m, 32 * qq, g);
                const V4 a1 = lds_kblock<F32>(Kt, LDT, 16 * kb + m, 32 * qq + 16, g);
                acc = mma<F32>::pair(acc, a0, a1, De[2 * qq], De[2 * qq + 1]);
            }
            S[kb] = acc;
        }
    }

    if (ST) {
        const size_t sb = ((size_t)bb * Hv + hv) * DK * DV;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) ST[sb + (size_t)(16 * kb + 4 * g + i) * DV + col] = S[kb][i];
    }
}

// T == 0: the final state is the initial state (or zero).
__global__ void state_copy_kernel(size_t n, const float *__restrict__ S0, float *__restrict__ ST) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        ST[i] = S0 ? S0[i] : 0.f;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_gate_prep(const PrefillArgs &p, const PrefillWorkspace &ws, hipStream_t s) {
    const int NC = (p.T + C - 1) / C;
    const long units = (long)p.B * p.Hv * NC;
    const unsigned blocks = (unsigned)((units + 3) / 4);
    hipLaunchKernelGGL(gate_prep_kernel, dim3(blocks), dim3(256), 0, s, p.B, p.T, p.Hv, NC, p.a,
                       p.b, p.A_log, p.dt_bias, ws.G, ws.beta);
    return hipGetLastError();
}

template <bool F32, typename TIn, int DK>
static hipError_t launch_chunk_local_t(const PrefillArgs &p, const PrefillWorkspace &ws, hipStream_t s) {
    typedef typename mma<F32>::E E;
    const int NC = (p.T + C - 1) / C;
    hipLaunchKernelGGL((chunk_local_kernel<F32, TIn, DK>), dim3(NC, p.Hk, p.B), dim3(256), 0, s,
                       p.B, p.T, p.Hk, p.Hv, NC, (const TIn *)p.q, (const TIn *)p.k, ws.G, ws.beta,
                       ws.tok, (E *)ws.apair, (E *)ws.qpair);
    return hipGetLastError();
}

hipError_t launch_chunk_local(const PrefillArgs &p, const PrefillWorkspace &ws, hipStream_t s) {
    if (p.f32) return p.Dk == 128 ? launch_chunk_local_t<true, float, 128>(p, ws, s)
                                   : launch_chunk_local_t<true, float, 64>(p, ws, s);
    return p.Dk == 128 ? launch_chunk_local_t<false, bf16_t, 128>(p, ws, s)
                       : launch_chunk_local_t<false, bf16_t, 64>(p, ws, s);
}

template <bool F32, typename TIn, int DK, int DV>
static hipError_t launch_scan_t(const PrefillArgs &p, const PrefillWorkspace &ws, hipStream_t s) {
    typedef typename mma<F32>::E E;
    const int NC = (p.T + C - 1) / C;
    const unsigned blocks = (unsigned)(p.B * p.Hv * (DV / 64));
    hipLaunchKernelGGL((state_scan_kernel<F32, TIn, DK, DV>), dim3(blocks), dim3(256), 0, s, p.B,
                       p.T, p.Hk, p.Hv, NC, p.scale, (const TIn *)p.q, (const TIn *)p.k,
                       (const TIn *)p.v, ws.tok, (const E *)ws.apair, (const E *)ws.qpair, p.S0,
                       (TIn *)p.out, p.ST);
    return hipGetLastError();
}

template <bool F32, typename TIn>
static hipError_t launch_scan_dt(const PrefillArgs &p, const PrefillWorkspace &ws, hipStream_t s) {
    if (p.Dk == 128 && p.Dv == 128) return launch_scan_t<F32, TIn, 128, 128>(p, ws, s);
    if (p.Dk == 128 && p.Dv == 64) return launch_scan_t<F32, TIn, 128, 64>(p, ws, s);
    if (p.Dk == 64 && p.Dv == 128) return launch_scan_t<F32, TIn, 64, 128>(p, ws, s);
    if (p.Dk == 64 && p.Dv == 64) return launch_scan_t<F32, TIn, 64, 64>(p, ws, s);
    return hipErrorInvalidValue;
}

hipError_t launch_state_scan(const PrefillArgs &p, const PrefillWorkspace &ws, hipStream_t s) {
    return p.f32 ? launch_scan_dt<true, float>(p, ws, s) : launch_scan_dt<false, bf16_t>(p, ws, s);
}

hipError_t launch_state_copy(const PrefillArgs &p, hipStream_t s) {
    if (!p.ST) return hipSuccess;
    const size_t n = (size_t)p.B * p.Hv * p.Dk * p.Dv;
    if (n == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(state_copy_kernel, dim3(blocks), dim3(256), 0, s, n, p.S0, p.ST);
    return hipGetLastError();
}

}  // namespace gdn
