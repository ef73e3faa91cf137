// bwd2.hip -- gradient of the Gated DeltaNet-2 chunked forward (zhichai.net,
// "Gated DeltaNet-2": sections "WY 形式" for the chunk form that is
// differentiated, "Gate-aware 反向传播" for the backward's requirement that the
// gate factors stay at the accumulation points: dA += dU Z^T, dA += dY Ebar^T).
//
// Per chunk of C = 64 tokens (n), value head and sequence, with G the in-chunk
// inclusive prefix of the channel-wise log decay, gamma = e^G, e = sigmoid(erase) k,
// z = sigmoid(write) v, qs = scale q:
//   Et = gamma . e, Qt = gamma . qs, Kh = (gamma_C / gamma) . k      (rows)
//   M[t][i]  = sum_c e_t k_i e^{G_t - G_i}  (i < t),   A = (I + M)^{-1}
//   Aq[t][i] = sum_c qs_t k_i e^{G_t - G_i} (i <= t)
//   R = Z - Et S_n,  U = A R,  O = Qt S_n + Aq U,  S_{n+1} = gamma_C . S_n + Kh^T U.
// Its adjoint, given dO and dS_{n+1}:
//   dU = Aq^T dO + Kh dS_{n+1};  dR = dZ = A^T dU
//   dS_n = gamma_C . dS_{n+1} + Qt^T dO - Et^T dR          (the reverse state scan)
//   dEt = -dR S_n^T,  dQt = dO S_n^T,  dKh = U dS_{n+1}^T,  dgamma_C = rowsum(dS_{n+1} . S_n)
//   dAq = tril(dO U^T),  dA = dU R^T = dU Z^T + dY Et^T (dY = -dU S_n^T),
//   dM = -strict_tril(A^T dA A^T)
// and through the pairwise decay: with E = e^{G_t - G_i},
//   de_t += sum_i dM_ti k_i E,  dqs_t += sum_i dAq_ti k_i E,
//   dk_i += sum_t (dM_ti e_t + dAq_ti qs_t) E,
//   dG_t += e_t de^M_t + qs_t dqs^A_t - k_t dk^P_t  (+ the image terms),
// then dg = reverse in-chunk prefix of dG, and the gates' own derivatives.
//
// Every quantity is float32.  The work is split over six launches:
//   g2b_prep       per chunk: gates, images, M and Aq, A = (I + M)^{-1}
//   g2b_fwd_scan   per (sequence, head, 32 value columns): S_n, R, U over the chunks
//   g2b_bwd_scan   the same slices in reverse: dS_{n+1}, dU, dR; dS_0
//   g2b_products   per chunk: dEt, dQt, dKh, dgamma_C, dAq, dM
//   g2b_local      per (chunk, 64 key channels): pairwise decay sums, gate chain
//   g2b_reduce     dq, dk over the value heads of a key head; dA_log over chunks
// Decay factors never exceed 1: a product e^{G_t - G_i} over a 16-token block
// pair below the diagonal is split at the block's first row r (i < r <= t) into
// e^{G_t - G_r} e^{G_r - G_i}; inside a diagonal block it is either taken
// directly or split at dyadic sub-blocks (first token of the second half).
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int C = 64;
constexpr float LOG2E = 1.4426950408889634f;

// acc += A(16 x K) B(K x 16), A(m, k) = a0[m * AM + k * AK], B(k, n) = b0[k * BK + n * BN]
// (K a multiple of 4; float32 MFMA, lane l supplies A[l%16][l/16], B[l/16][l%16]).
// Fully unrolled so that the operand reads are issued ahead of the MFMAs.
template <int K, int AM, int AK, int BK, int BN>
__device__ __forceinline__ void mma(f4 &acc, const float *a0, const float *b0) {
    const int l = threadIdx.x & 63, r = l & 15, g = l >> 4;
    const float *pa = a0 + r * AM + g * AK, *pb = b0 + g * BK + r * BN;
#pragma unroll
    for (int k = 0; k < K; k += 4) acc = mfma_f32_k4(pa[k * AK], pb[k * BK], acc);
}

// ROWS x COLS float32 block (row-major, contiguous) into LDS rows of stride LS,
// times f.  Compile-time trip counts: each thread issues its loads in batches of
// 8 before storing them, so the global latency is paid once per batch.
template <int ROWS, int COLS, int LS, int NT = 256>
__device__ __forceinline__ void lds_load(float *dst, const float *__restrict__ src, float f = 1.f) {
    constexpr int N = ROWS * COLS / 4, PER = N / NT, BT = PER < 8 ? PER : 8;
    static_assert(N % NT == 0 && PER % BT == 0, "block size");
#pragma unroll
    for (int b0 = 0; b0 < PER; b0 += BT) {
        f4 x[BT];
#pragma unroll
        for (int j = 0; j < BT; ++j)
            x[j] = *reinterpret_cast<const f4 *>(src + (size_t)(threadIdx.x + (b0 + j) * NT) * 4);
#pragma unroll
        for (int j = 0; j < BT; ++j) {
            const int i = threadIdx.x + (b0 + j) * NT, r = i / (COLS / 4), c = (i % (COLS / 4)) * 4;
            *reinterpret_cast<f4 *>(dst + r * LS + c) = x[j] * f;
        }
    }
}

// 8 bfloat16 values to float32
__device__ __forceinline__ void bf8_to_f32(const u16x8 x, f4 &lo, f4 &hi) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        lo[j] = bf16_to_f32(x[j]);
        hi[j] = bf16_to_f32(x[j + 4]);
    }
}

// A ROWS x COLS float32 tile (row-major, contiguous) held in registers between
// its global load and its LDS store: the scans load the next chunk's operands
// while computing the current one.
template <int ROWS, int COLS, int NT = 256> struct RegTile {
    static constexpr int PER = ROWS * COLS / 4 / NT;
    static_assert(ROWS * COLS / 4 % NT == 0, "tile size");
    f4 x[PER];
    __device__ __forceinline__ void load(const float *__restrict__ src) {
#pragma unroll
        for (int j = 0; j < PER; ++j) x[j] = *reinterpret_cast<const f4 *>(src + (size_t)(threadIdx.x + j * NT) * 4);
    }
    template <int LS> __device__ __forceinline__ void store(float *dst, float f = 1.f) const {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int i = threadIdx.x + j * NT, r = i / (COLS / 4), c = (i % (COLS / 4)) * 4;
            *reinterpret_cast<f4 *>(dst + r * LS + c) = x[j] * f;
        }
    }
};

// 2^x on the hardware unit (arguments here are <= 0: every decay factor is at most 1)
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ size_t unit_of(int bb, int hv, int n, int Hv, int NC) {
    return ((size_t)bb * Hv + hv) * NC + n;
}

// ---------------------------------------------------------------------------
// g2b_prep: one work-group of 4 waves per (sequence, value head, chunk)
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(256) void g2b_prep(Bwd2Args p, Bwd2Workspace ws) {
    constexpr int LS = DK + 4;  // conflict-free for lanes (row = l%16, col = l/16)
    __shared__ __attribute__((aligned(16))) float sm[4 * C * LS + C];
    float *Gs = sm, *Es = Gs + C * LS, *Qs = Es + C * LS, *Ks = Qs + C * LS, *dd = Ks + C * LS;
    float *Ms = Es, *As = Qs, *Xt = Ks;  // after the tiles: M, A (stride 68), 4 x [16][48] scratch

    const int u = blockIdx.x, NC = p.NC;
    const int n = u % NC, hv = (u / NC) % p.Hv, bb = u / (NC * p.Hv), hk = hv / (p.Hv / p.Hk);
    const int t0 = n * C, L = min(C, p.T - t0);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, rr = lane & 15, gg = lane >> 4;
    const uint16_t *v = reinterpret_cast<const uint16_t *>(p.v), *wr = reinterpret_cast<const uint16_t *>(p.write);

    // 1. gates: G (log2 units, 0 past T), e = sigmoid(erase) k, qs = scale q, k; z to the workspace.
    //    Thread = (4 channels, a group of RPT consecutive rows); rows past T read the last
    //    token (L >= 1) and are zeroed, so every load is unconditional.  The in-chunk prefix
    //    of g is taken over the thread's rows, then the totals of the earlier row groups
    //    are added.
    constexpr int NQ = DK / 4, NRG = 256 / NQ, RPT = C / NRG;
    __shared__ float tot[NRG * DK];
    {
        const bf16_t *qb = reinterpret_cast<const bf16_t *>(p.q), *kb = reinterpret_cast<const bf16_t *>(p.k);
        const bf16_t *ab = reinterpret_cast<const bf16_t *>(p.a), *eb = reinterpret_cast<const bf16_t *>(p.erase);
        const int c = (tid % NQ) * 4, rg = tid / NQ;
        const f4 al = *reinterpret_cast<const f4 *>(p.A_log + (size_t)hv * DK + c);
        f4 rate;
#pragma unroll
        for (int j = 0; j < 4; ++j) rate[j] = -exp_fast(al[j]) * LOG2E;
        f4 run = {0, 0, 0, 0}, gr[RPT];
#pragma unroll
        for (int x = 0; x < RPT; ++x) {
            const int t = rg * RPT + x, tl = min(t, L - 1);
            const size_t kq = (((size_t)bb * p.T + t0 + tl) * p.Hk + hk) * DK + c;
            const size_t ka = (((size_t)bb * p.T + t0 + tl) * p.Hv + hv) * DK + c;
            const f4 kk = ld4(kb, kq), qq = ld4(qb, kq), aa = ld4(ab, ka), ee = ld4(eb, ka);
            const float on = t < L ? 1.f : 0.f;
            f4 ev, qv, kv;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                run[j] += rate[j] * softplus_fast(aa[j]) * on;
                ev[j] = sigmoid_fast(ee[j]) * kk[j] * on;
                qv[j] = p.scale * qq[j] * on;
                kv[j] = kk[j] * on;
            }
            gr[x] = run;
            *reinterpret_cast<f4 *>(Es + t * LS + c) = ev;
            *reinterpret_cast<f4 *>(Qs + t * LS + c) = qv;
            *reinterpret_cast<f4 *>(Ks + t * LS + c) = kv;
        }
        *reinterpret_cast<f4 *>(tot + rg * DK + c) = run;
        __syncthreads();
        f4 off = {0, 0, 0, 0};
        for (int x = 0; x < rg; ++x) off += *reinterpret_cast<const f4 *>(tot + x * DK + c);
#pragma unroll
        for (int x = 0; x < RPT; ++x) *reinterpret_cast<f4 *>(Gs + (rg * RPT + x) * LS + c) = gr[x] + off;
    }
    float *Zu = ws.Z + (size_t)u * C * DV;
#pragma unroll
    for (int it = 0; it < C * DV / 8 / 256; ++it) {
        const int i = tid + 256 * it, t = i / (DV / 8), j = (i % (DV / 8)) * 8, tl = min(t, L - 1);
        const size_t kv = (((size_t)bb * p.T + t0 + tl) * p.Hv + hv) * DV + j;
        f4 vl, vh, wl, wh;
        bf8_to_f32(*reinterpret_cast<const u16x8 *>(v + kv), vl, vh);
        bf8_to_f32(*reinterpret_cast<const u16x8 *>(wr + kv), wl, wh);
        const float on = t < L ? 1.f : 0.f;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            vl[x] = sigmoid_fast(wl[x]) * vl[x] * on;
            vh[x] = sigmoid_fast(wh[x]) * vh[x] * on;
        }
        *reinterpret_cast<f4 *>(Zu + t * DV + j) = vl;
        *reinterpret_cast<f4 *>(Zu + t * DV + j + 4) = vh;
    }
    __syncthreads();
    // 3. images, gamma_C and the diagonal of Aq (q_t . k_t, no decay)
    {
        const size_t ub = (size_t)u * C * DK;
        for (int i = tid; i < C * DK / 4; i += 256) {
            const int t = i / (DK / 4), c = (i % (DK / 4)) * 4;
            const f4 G = *reinterpret_cast<const f4 *>(Gs + t * LS + c);
            const f4 GC = *reinterpret_cast<const f4 *>(Gs + (C - 1) * LS + c);
            f4 eg, kg;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                eg[j] = ex2(G[j]);
                kg[j] = ex2(GC[j] - G[j]);
            }
            *reinterpret_cast<f4 *>(ws.Et + ub + t * DK + c) = *reinterpret_cast<const f4 *>(Es + t * LS + c) * eg;
            *reinterpret_cast<f4 *>(ws.Qt + ub + t * DK + c) = *reinterpret_cast<const f4 *>(Qs + t * LS + c) * eg;
            *reinterpret_cast<f4 *>(ws.Kh + ub + t * DK + c) = *reinterpret_cast<const f4 *>(Ks + t * LS + c) * kg;
        }
        for (int c = tid; c < DK; c += 256) ws.gC[(size_t)u * DK + c] = ex2(Gs[(C - 1) * LS + c]);
        if (tid < C) {
            float s = 0.f;
            for (int c = 0; c < DK; ++c) s += Qs[tid * LS + c] * Ks[tid * LS + c];
            dd[tid] = s;
        }
    }
    __syncthreads();
    // 4. M and Aq.  Tiles below the diagonal (bt > bi), reference row r = 16 bt:
    //    sum_c [e_t e^{G_t - G_r}] [k_i e^{G_r - G_i}].  Wave w takes tiles w, w + 4.
    constexpr int OBT[6] = {1, 2, 2, 3, 3, 3}, OBI[6] = {0, 0, 1, 0, 1, 2};
    f4 mO[2], qO[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        mO[x] = qO[x] = f4{0, 0, 0, 0};
        const int ti = w + 4 * x;
        if (ti < 6) {
            const int bt = OBT[ti], bi = OBI[ti], r = 16 * bt, t = 16 * bt + rr, i = 16 * bi + rr;
#pragma unroll 8
            for (int c0 = 0; c0 < DK; c0 += 4) {
                const int c = c0 + gg;
                const float Gr = Gs[r * LS + c];
                const float ft = ex2(Gs[t * LS + c] - Gr), b = Ks[i * LS + c] * ex2(Gr - Gs[i * LS + c]);
                mO[x] = mfma_f32_k4(Es[t * LS + c] * ft, b, mO[x]);
                qO[x] = mfma_f32_k4(Qs[t * LS + c] * ft, b, qO[x]);
            }
        }
    }
    //    Diagonal tile w: dyadic levels (half sizes 8, 4, 2, 1); a pair (t > i) of
    //    the tile belongs to the level whose 2h-block holds both with i in the
    //    first and t in the second half; reference = first token of that half.
    f4 mD = {0, 0, 0, 0}, qD = {0, 0, 0, 0};
    {
        const int base = 16 * w, t = base + rr, i = base + rr;
#pragma unroll
        for (int h = 8; h >= 1; h >>= 1) {
            const bool tsec = (rr & h) != 0;
            const int rt = base + (rr & ~(h - 1)), ri = base + ((rr | h) & ~(h - 1));
            f4 aM = {0, 0, 0, 0}, aQ = {0, 0, 0, 0};
#pragma unroll 8
            for (int c0 = 0; c0 < DK; c0 += 4) {
                const int c = c0 + gg;
                float ae = 0.f, aq = 0.f, b = 0.f;
                if (tsec) {
                    const float ft = ex2(Gs[t * LS + c] - Gs[rt * LS + c]);
                    ae = Es[t * LS + c] * ft;
                    aq = Qs[t * LS + c] * ft;
                } else {
                    b = Ks[i * LS + c] * ex2(Gs[ri * LS + c] - Gs[i * LS + c]);
                }
                aM = mfma_f32_k4(ae, b, aM);
                aQ = mfma_f32_k4(aq, b, aQ);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int tl = 4 * gg + s;
                if (((tl ^ rr) & ~(2 * h - 1)) == 0 && (tl & h) && !(rr & h)) {
                    mD[s] += aM[s];
                    qD[s] += aQ[s];
                }
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
            if (4 * gg + s == rr) qD[s] += dd[base + rr];
    }
    __syncthreads();  // Es, Qs, Ks are reused below
    // Aq to the workspace (zero above the diagonal); M into LDS (zero on and above)
    {
        float *Aqu = ws.Aq + (size_t)u * C * C;
        for (int i = tid; i < C * 68; i += 256) Ms[i] = 0.f;
        __syncthreads();
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int ti = w + 4 * x;
            if (ti < 6) {
                const int bt = OBT[ti], bi = OBI[ti];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int t = 16 * bt + 4 * gg + s, i = 16 * bi + rr;
                    Ms[t * 68 + i] = mO[x][s];
                    Aqu[t * C + i] = qO[x][s];
                    Aqu[i * C + t] = 0.f;  // the mirrored tile above the diagonal
                }
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int t = 16 * w + 4 * gg + s, i = 16 * w + rr;
            Ms[t * 68 + i] = mD[s];
            Aqu[t * C + i] = qD[s];
        }
    }
    __syncthreads();
    // 5. A = (I + M)^{-1}: diagonal 16 x 16 blocks by forward substitution (wave w,
    //    lane j < 16 owns column j of block w), then block rows 1..3:
    //    A_bj = -A_bb sum_{m=j}^{b-1} M_bm A_mj.
    if (lane < 16) {
        const int base = 16 * w, j = lane;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float s = (t == j) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < t; ++i) s -= Ms[(base + t) * 68 + base + i] * x[i];
            x[t] = s;
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) As[(base + t) * 68 + base + j] = x[t];
    }
    // zero the blocks above the diagonal of A
    for (int i = tid; i < C * C; i += 256) {
        const int t = i / C, c = i % C;
        if ((c >> 4) > (t >> 4)) As[t * 68 + c] = 0.f;
    }
    __syncthreads();
    for (int b = 1; b < 4; ++b) {
        if (w < b) {
            f4 X = {0, 0, 0, 0};
            for (int m = w; m < b; ++m) mma<16, 68, 1, 68, 1>(X, Ms + 16 * b * 68 + 16 * m, As + 16 * m * 68 + 16 * w);
#pragma unroll
            for (int s = 0; s < 4; ++s) Xt[w * 16 * 48 + (4 * gg + s) * 48 + rr] = X[s];
        }
        __syncthreads();
        if (w < b) {
            f4 Y = {0, 0, 0, 0};
            mma<16, 68, 1, 48, 1>(Y, As + 16 * b * 68 + 16 * b, Xt + w * 16 * 48);
#pragma unroll
            for (int s = 0; s < 4; ++s) As[(16 * b + 4 * gg + s) * 68 + 16 * w + rr] = -Y[s];
        }
        __syncthreads();
    }
    float *Au = ws.A + (size_t)u * C * C;
    for (int i = tid; i < C * C / 4; i += 256) {
        const int t = i / (C / 4), c = (i % (C / 4)) * 4;
        *reinterpret_cast<f4 *>(Au + t * C + c) = *reinterpret_cast<const f4 *>(As + t * 68 + c);
    }
}

// ---------------------------------------------------------------------------
// g2b_fwd_scan: one work-group per (sequence, value head, 32 value columns);
// wave w holds the state tiles (c-blocks 2w', j-blocks) as MFMA accumulators.
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(256) void g2b_fwd_scan(Bwd2Args p, Bwd2Workspace ws) {
    constexpr int LE = DK + 4, LK = DK + 16, LA = 68, LB = 48, NS = DV / 32, NT = DK / 32;
    __shared__ __attribute__((aligned(16))) float Ets[C * LE], Khs[C * LK], As[C * LA], Ss[DK * LB], Rs[C * LB],
        Us[C * LB];
    const int js = blockIdx.x % NS, hv = (blockIdx.x / NS) % p.Hv, bb = blockIdx.x / (NS * p.Hv), j0 = 32 * js;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, rr = lane & 15, gg = lane >> 4, NC = p.NC;
    f4 S[NT];
#pragma unroll
    for (int x = 0; x < NT; ++x) {
        const int id = w * NT + x, cb = id >> 1, jb = id & 1;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int c = 16 * cb + 4 * gg + s, j = 16 * jb + rr;
            S[x][s] = p.S0 ? p.S0[(((size_t)bb * p.Hv + hv) * DK + c) * DV + j0 + j] : 0.f;
            Ss[c * LB + j] = S[x][s];
        }
    }
    for (int n = 0; n < NC; ++n) {
        const size_t u = unit_of(bb, hv, n, p.Hv, NC);
        float *Snu = ws.Sn + u * DK * DV;
#pragma unroll
        for (int x = 0; x < NT; ++x) {
            const int id = w * NT + x, cb = id >> 1, jb = id & 1;
#pragma unroll
            for (int s = 0; s < 4; ++s) Snu[(16 * cb + 4 * gg + s) * DV + j0 + 16 * jb + rr] = S[x][s];
        }
        // this lane's Z elements and decay factors, loaded ahead of the staging
        const float *Zu = ws.Z + u * C * DV, *gCu = ws.gC + u * DK;
        float zr[2][4], gcr[NT][4];
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int s = 0; s < 4; ++s) zr[jb][s] = Zu[(16 * w + 4 * gg + s) * DV + j0 + 16 * jb + rr];
#pragma unroll
        for (int x = 0; x < NT; ++x)
#pragma unroll
            for (int s = 0; s < 4; ++s) gcr[x][s] = gCu[16 * ((w * NT + x) >> 1) + 4 * gg + s];
        lds_load<C, DK, LE>(Ets, ws.Et + u * C * DK);
        lds_load<C, DK, LK>(Khs, ws.Kh + u * C * DK);
        lds_load<C, C, LA>(As, ws.A + u * C * C);
        __syncthreads();
        // R = Z - Et S (rows of block w)
        float *Ru = ws.R + u * C * DV, *Uu = ws.U + u * C * DV;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            f4 acc = {0, 0, 0, 0};
            mma<DK, LE, 1, LB, 1>(acc, Ets + 16 * w * LE, Ss + 16 * jb);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int t = 16 * w + 4 * gg + s, j = 16 * jb + rr;
                const float rv = zr[jb][s] - acc[s];
                Rs[t * LB + j] = rv;
                Ru[t * DV + j0 + j] = rv;
            }
        }
        __syncthreads();
        // U = A R (A lower triangular: columns up to the block's last row)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            f4 acc = {0, 0, 0, 0};
            mma<C, LA, 1, LB, 1>(acc, As + 16 * w * LA, Rs + 16 * jb);  // A is zero above the diagonal
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int t = 16 * w + 4 * gg + s, j = 16 * jb + rr;
                Us[t * LB + j] = acc[s];
                Uu[t * DV + j0 + j] = acc[s];
            }
        }
        __syncthreads();
        // S = gamma_C . S + Kh^T U
#pragma unroll
        for (int x = 0; x < NT; ++x) {
            const int id = w * NT + x, cb = id >> 1, jb = id & 1;
#pragma unroll
            for (int s = 0; s < 4; ++s) S[x][s] *= gcr[x][s];
            mma<C, 1, LK, LB, 1>(S[x], Khs + 16 * cb, Us + 16 * jb);
#pragma unroll
            for (int s = 0; s < 4; ++s) Ss[(16 * cb + 4 * gg + s) * LB + 16 * jb + rr] = S[x][s];
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// g2b_bwd_scan: the same slices, chunks in reverse; dS in MFMA accumulators.
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(256) void g2b_bwd_scan(Bwd2Args p, Bwd2Workspace ws) {
    constexpr int LQ = 80, LKA = DK + 4, LKB = DK + 16, LB = 48, NS = DV / 32, NT = DK / 32;
    // bA: A_qk, then A; bK1: Kh (stride LKA), then -Et (stride LKB); bK2: Qt
    __shared__ __attribute__((aligned(16))) float bA[C * LQ], bK1[C * LKB], bK2[C * LKB], Os[C * LB],
        dSs[DK * LB], dUs[C * LB], dRs[C * LB];
    const int js = blockIdx.x % NS, hv = (blockIdx.x / NS) % p.Hv, bb = blockIdx.x / (NS * p.Hv), j0 = 32 * js;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, rr = lane & 15, gg = lane >> 4, NC = p.NC;
    const uint16_t *dout = reinterpret_cast<const uint16_t *>(p.dout);
    f4 dS[NT];
#pragma unroll
    for (int x = 0; x < NT; ++x) {
        const int id = w * NT + x, cb = id >> 1, jb = id & 1;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int c = 16 * cb + 4 * gg + s, j = 16 * jb + rr;
            dS[x][s] = p.dST ? p.dST[(((size_t)bb * p.Hv + hv) * DK + c) * DV + j0 + j] : 0.f;
            dSs[c * LB + j] = dS[x][s];
        }
    }
    // dO slice of chunk n: 64 rows x 32 columns, 8 per thread (rows past T read the last
    // token and are zeroed when stored)
    const int ot = tid >> 2, oj = (tid & 3) * 8;
    auto load_do = [&](int n) {
        const int L = min(C, p.T - n * C), tl = min(ot, L - 1);
        return *reinterpret_cast<const u16x8 *>(dout + (((size_t)bb * p.T + n * C + tl) * p.Hv + hv) * DV + j0 + oj);
    };
    auto store_do = [&](const u16x8 x, int n) {
        const int L = min(C, p.T - n * C);
        f4 lo, hi;
        bf8_to_f32(x, lo, hi);
        const float on = ot < L ? 1.f : 0.f;
        *reinterpret_cast<f4 *>(Os + ot * LB + oj) = lo * on;
        *reinterpret_cast<f4 *>(Os + ot * LB + oj + 4) = hi * on;
    };
    // staged for the chunk about to run: A_qk in bA, Kh in bK1, dO in Os
    RegTile<C, C> rAq, rA;
    RegTile<C, DK> rKh, rQ, rE;
    u16x8 rdo;
    {
        const size_t u = unit_of(bb, hv, NC - 1, p.Hv, NC);
        rAq.load(ws.Aq + u * C * C);
        rKh.load(ws.Kh + u * C * DK);
        rdo = load_do(NC - 1);
        rAq.template store<LQ>(bA);
        rKh.template store<LKA>(bK1);
        store_do(rdo, NC - 1);
    }
    for (int n = NC - 1; n >= 0; --n) {
        const size_t u = unit_of(bb, hv, n, p.Hv, NC);
        float *dS1u = ws.dS1 + u * DK * DV;
#pragma unroll
        for (int x = 0; x < NT; ++x) {
            const int id = w * NT + x, cb = id >> 1, jb = id & 1;
#pragma unroll
            for (int s = 0; s < 4; ++s) dS1u[(16 * cb + 4 * gg + s) * DV + j0 + 16 * jb + rr] = dS[x][s];
        }
        float gcr[NT][4];
#pragma unroll
        for (int x = 0; x < NT; ++x)
#pragma unroll
            for (int s = 0; s < 4; ++s) gcr[x][s] = ws.gC[u * DK + 16 * ((w * NT + x) >> 1) + 4 * gg + s];
        __syncthreads();
        // this chunk's A, Qt, Et in flight while dU is computed
        rA.load(ws.A + u * C * C);
        rQ.load(ws.Qt + u * C * DK);
        rE.load(ws.Et + u * C * DK);
        // dU = Aq^T dO + Kh dS  (Aq is zero above the diagonal)
        float *dUu = ws.dU + u * C * DV, *dRu = ws.dR + u * C * DV;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            f4 acc = {0, 0, 0, 0};
            mma<C, 1, LQ, LB, 1>(acc, bA + 16 * w, Os + 16 * jb);
            mma<DK, LKA, 1, LB, 1>(acc, bK1 + 16 * w * LKA, dSs + 16 * jb);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int t = 16 * w + 4 * gg + s, j = 16 * jb + rr;
                dUs[t * LB + j] = acc[s];
                dUu[t * DV + j0 + j] = acc[s];
            }
        }
        __syncthreads();
        rA.template store<LQ>(bA);
        rQ.template store<LKB>(bK2);
        rE.template store<LKB>(bK1, -1.f);
        // the next chunk's A_qk, Kh and dO in flight while this one finishes
        if (n > 0) {
            const size_t un = u - 1;
            rAq.load(ws.Aq + un * C * C);
            rKh.load(ws.Kh + un * C * DK);
            rdo = load_do(n - 1);
        }
        __syncthreads();
        // dR = A^T dU;  dS = gamma_C . dS + Qt^T dO
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            f4 acc = {0, 0, 0, 0};
            mma<C, 1, LQ, LB, 1>(acc, bA + 16 * w, dUs + 16 * jb);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int t = 16 * w + 4 * gg + s, j = 16 * jb + rr;
                dRs[t * LB + j] = acc[s];
                dRu[t * DV + j0 + j] = acc[s];
            }
        }
#pragma unroll
        for (int x = 0; x < NT; ++x) {
            const int id = w * NT + x, cb = id >> 1, jb = id & 1;
#pragma unroll
            for (int s = 0; s < 4; ++s) dS[x][s] *= gcr[x][s];
            mma<C, 1, LKB, LB, 1>(dS[x], bK2 + 16 * cb, Os + 16 * jb);
        }
        __syncthreads();
        // dS -= Et^T dR  (bK1 holds -Et)
#pragma unroll
        for (int x = 0; x < NT; ++x) {
            const int id = w * NT + x, cb = id >> 1, jb = id & 1;
            mma<C, 1, LKB, LB, 1>(dS[x], bK1 + 16 * cb, dRs + 16 * jb);
#pragma unroll
            for (int s = 0; s < 4; ++s) dSs[(16 * cb + 4 * gg + s) * LB + 16 * jb + rr] = dS[x][s];
        }
        __syncthreads();
        if (n > 0) {
            rAq.template store<LQ>(bA);
            rKh.template store<LKA>(bK1);
            store_do(rdo, n - 1);
        }
    }
    if (p.dS0) {
#pragma unroll
        for (int x = 0; x < NT; ++x) {
            const int id = w * NT + x, cb = id >> 1, jb = id & 1;
#pragma unroll
            for (int s = 0; s < 4; ++s)
                p.dS0[(((size_t)bb * p.Hv + hv) * DK + 16 * cb + 4 * gg + s) * DV + j0 + 16 * jb + rr] = dS[x][s];
        }
    }
}

// ---------------------------------------------------------------------------
// g2b_products: one work-group per chunk.  Wave w owns the rows of block w.
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(256) void g2b_products(Bwd2Args p, Bwd2Workspace ws) {
    constexpr int LV = DV + 4, R1 = (DK * LV > 2 * C * 80) ? DK * LV : 2 * C * 80;
    __shared__ __attribute__((aligned(16))) float r1[R1], b1[C * LV], b2[C * LV];
    const int u = blockIdx.x, NC = p.NC;
    const int n = u % NC, hv = (u / NC) % p.Hv, bb = u / (NC * p.Hv);
    const int t0 = n * C, L = min(C, p.T - t0);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, rr = lane & 15, gg = lane >> 4;
    const size_t uC = (size_t)u * C;
    const uint16_t *dout = reinterpret_cast<const uint16_t *>(p.dout);

    // phase 1: dEt = -dR Sn^T, dQt = dO Sn^T, dgamma_C = rowsum(dS1 . Sn)
    {
        // dO: 8 values per load (rows past T read the last token, zeroed)
        u16x8 xo[C * DV / 8 / 256];
#pragma unroll
        for (int it = 0; it < C * DV / 8 / 256; ++it) {
            const int i = tid + 256 * it, t = i / (DV / 8), j = (i % (DV / 8)) * 8, tl = min(t, L - 1);
            xo[it] = *reinterpret_cast<const u16x8 *>(dout + (((size_t)bb * p.T + t0 + tl) * p.Hv + hv) * DV + j);
        }
        lds_load<DK, DV, LV>(r1, ws.Sn + (size_t)u * DK * DV);
        lds_load<C, DV, LV>(b1, ws.dR + uC * DV, -1.f);
#pragma unroll
        for (int it = 0; it < C * DV / 8 / 256; ++it) {
            const int i = tid + 256 * it, t = i / (DV / 8), j = (i % (DV / 8)) * 8;
            f4 lo, hi;
            bf8_to_f32(xo[it], lo, hi);
            const float on = t < L ? 1.f : 0.f;
            *reinterpret_cast<f4 *>(b2 + t * LV + j) = lo * on;
            *reinterpret_cast<f4 *>(b2 + t * LV + j + 4) = hi * on;
        }
    }
    __syncthreads();
    for (int cb = 0; cb < DK / 16; ++cb) {
        f4 e = {0, 0, 0, 0}, q = {0, 0, 0, 0};
        mma<DV, LV, 1, 1, LV>(e, b1 + 16 * w * LV, r1 + 16 * cb * LV);
        mma<DV, LV, 1, 1, LV>(q, b2 + 16 * w * LV, r1 + 16 * cb * LV);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const size_t o = (uC + 16 * w + 4 * gg + s) * DK + 16 * cb + rr;
            ws.dEt[o] = e[s];
            ws.dQt[o] = q[s];
        }
    }
    if (tid < 2 * DK) {
        const int c = tid >> 1, h = tid & 1;
        const float *d1 = ws.dS1 + ((size_t)u * DK + c) * DV + h * (DV / 2);
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < DV / 2; j += 4) {
            const f4 x = *reinterpret_cast<const f4 *>(d1 + j), y = *reinterpret_cast<const f4 *>(r1 + c * LV + h * (DV / 2) + j);
            s += x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
        }
        s += __shfl_xor(s, 1);
        if (!h) ws.dgC[(size_t)u * DK + c] = s;
    }
    __syncthreads();
    // phase 2: dKh = U dS1^T, dAq = tril(dO U^T)
    lds_load<DK, DV, LV>(r1, ws.dS1 + (size_t)u * DK * DV);
    lds_load<C, DV, LV>(b1, ws.U + uC * DV);
    __syncthreads();
    for (int cb = 0; cb < DK / 16; ++cb) {
        f4 acc = {0, 0, 0, 0};
        mma<DV, LV, 1, 1, LV>(acc, b1 + 16 * w * LV, r1 + 16 * cb * LV);
#pragma unroll
        for (int s = 0; s < 4; ++s) ws.dKh[(uC + 16 * w + 4 * gg + s) * DK + 16 * cb + rr] = acc[s];
    }
    float *dAqu = ws.dAq + uC * C;
    for (int ib = 0; ib < 4; ++ib) {
        f4 acc = {0, 0, 0, 0};
        if (ib <= w) mma<DV, LV, 1, 1, LV>(acc, b2 + 16 * w * LV, b1 + 16 * ib * LV);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int t = 16 * w + 4 * gg + s, i = 16 * ib + rr;
            dAqu[t * C + i] = i <= t ? acc[s] : 0.f;
        }
    }
    __syncthreads();
    // phase 3: dA = dU R^T; X = A^T dA; dM = -strict_tril(X A^T)
    float *dAs = r1, *A80 = r1 + C * 80, *A68 = b1, *Xs = b2;
    lds_load<C, DV, LV>(b1, ws.R + uC * DV);
    lds_load<C, DV, LV>(b2, ws.dU + uC * DV);
    lds_load<C, C, 80>(A80, ws.A + uC * C);
    __syncthreads();
    f4 dA[4];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
        dA[ib] = f4{0, 0, 0, 0};
        mma<DV, LV, 1, 1, LV>(dA[ib], b2 + 16 * w * LV, b1 + 16 * ib * LV);
    }
    __syncthreads();
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int s = 0; s < 4; ++s) dAs[(16 * w + 4 * gg + s) * 80 + 16 * ib + rr] = dA[ib][s];
    lds_load<C, C, 68>(A68, ws.A + uC * C);
    __syncthreads();
    // X[i][s] = sum_t A[t][i] dA[t][s] (A[t][i] = 0 for t < i): rows i of block w
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
        f4 acc = {0, 0, 0, 0};
        mma<C, 1, 80, 80, 1>(acc, A80 + 16 * w, dAs + 16 * sb);
        dA[sb] = acc;  // reuse the registers for X
    }
    __syncthreads();  // Xs aliases b2, read by nobody now; A68 stays
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
        for (int s = 0; s < 4; ++s) Xs[(16 * w + 4 * gg + s) * 68 + 16 * sb + rr] = dA[sb][s];
    __syncthreads();
    // dM[i][q] = -sum_s X[i][s] A[q][s] (A[q][s] = 0 for s > q), strictly lower
    float *dMu = ws.dM + uC * C;
    for (int qb = 0; qb < 4; ++qb) {
        f4 acc = {0, 0, 0, 0};
        if (qb <= w) mma<C, 68, 1, 1, 68>(acc, Xs + 16 * w * 68, A68 + 16 * qb * 68);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int i = 16 * w + 4 * gg + s, qq = 16 * qb + rr;
            dMu[i * C + qq] = qq < i ? -acc[s] : 0.f;
        }
    }
}

// ---------------------------------------------------------------------------
// g2b_local: one work-group of 8 waves per (chunk, 64 key channels).  Wave w
// owns rows 8w .. 8w+7, half of 16-token block b = w/2: first the block pairs
// below the diagonal on the matrix cores for block b and two of its four
// 16-channel tiles (rows t of block b against every earlier block, rows i of
// block b against every later block), then the pairs inside block b that its
// own rows take part in, on the vector unit (lane = channel), then the chain
// rule for its rows.
// ---------------------------------------------------------------------------
constexpr int LOCAL_NT = 512;

template <int DK, int DV>
__global__ __launch_bounds__(LOCAL_NT) void g2b_local(Bwd2Args p, Bwd2Workspace ws) {
    constexpr int CG = DK / 64, NW = LOCAL_NT / 64;
    __shared__ __attribute__((aligned(16))) float Gs[C * 64], Ks[C * 64], Es[C * 64], Qs[C * 64], dMs[C * C],
        dAqs[C * C], Te[C * 64], Tq[C * 64], Ik[C * 64], blk[NW * 64], gcp[NW * 64], alp[NW * 64];
    const int cg = blockIdx.x % CG, u = blockIdx.x / CG, NC = p.NC;
    const int n = u % NC, hv = (u / NC) % p.Hv, bb = u / (NC * p.Hv), hk = hv / (p.Hv / p.Hk);
    const int t0 = n * C, L = min(C, p.T - t0);
    const int tid = threadIdx.x, w = tid >> 6, cl = tid & 63, c = 64 * cg + cl, rr = cl & 15, gg = cl >> 4;
    const int b = w >> 1, half = w & 1, r0 = 8 * w;  // block, half of it, first own row
    const uint16_t *q = reinterpret_cast<const uint16_t *>(p.q), *k = reinterpret_cast<const uint16_t *>(p.k);
    const uint16_t *a = reinterpret_cast<const uint16_t *>(p.a), *er = reinterpret_cast<const uint16_t *>(p.erase);
    const float Al = p.A_log[(size_t)hv * DK + c], rate = exp_fast(Al);

    // inputs of the chain rule, loaded first so that their latency overlaps the pair sums
    const size_t ub = (size_t)u * C * DK;
    float pdE[8], pdQ[8], pdK[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
        pdE[x] = ws.dEt[ub + (r0 + x) * DK + c];
        pdQ[x] = ws.dQt[ub + (r0 + x) * DK + c];
        pdK[x] = ws.dKh[ub + (r0 + x) * DK + c];
    }
    const float pgC = ws.dgC[(size_t)u * DK + c];

    // gates of the wave's rows; the in-chunk prefix of g runs over them, then the
    // totals of the earlier row groups are added
    float grun = 0.f, gpre[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
        const int t = r0 + x, tl = min(t, L - 1);
        const size_t kq = (((size_t)bb * p.T + t0 + tl) * p.Hk + hk) * DK + c;
        const size_t ka = (((size_t)bb * p.T + t0 + tl) * p.Hv + hv) * DK + c;
        const float on = t < L ? 1.f : 0.f;
        const float kv = bf16_to_f32(k[kq]) * on;
        grun += -rate * softplus_fast(bf16_to_f32(a[ka])) * LOG2E * on;
        const float ev = sigmoid_fast(bf16_to_f32(er[ka])) * kv;
        const float qv = p.scale * bf16_to_f32(q[kq]) * on;
        gpre[x] = grun;
        Ks[t * 64 + cl] = kv;
        Es[t * 64 + cl] = ev;
        Qs[t * 64 + cl] = qv;
    }
    blk[w * 64 + cl] = grun;
    lds_load<C, C, C, LOCAL_NT>(dMs, ws.dM + (size_t)u * C * C);
    lds_load<C, C, C, LOCAL_NT>(dAqs, ws.dAq + (size_t)u * C * C);
    __syncthreads();
    {
        float off = 0.f;
        for (int x = 0; x < w; ++x) off += blk[x * 64 + cl];
#pragma unroll
        for (int x = 0; x < 8; ++x) Gs[(r0 + x) * 64 + cl] = gpre[x] + off;
    }
    __syncthreads();

    // block pairs below the diagonal, 16 channels at a time (MFMA: lane supplies
    // A[rr][gg], B[gg][rr]; accumulator element s is row 4 gg + s, channel rr).
    //   rows t of block b, reference r = 16 b (i < r <= t):
    //     de_t  = e^{G_t - G_r} sum_{i < r} dM_ti  k_i e^{G_r - G_i}, dqs_t likewise with dAq
    //   rows i of block b, each later block b2 with reference r = 16 b2:
    //     dk_i += e^{G_r - G_i} sum_{t in b2} dM_ti e_t e^{G_t - G_r} + dAq_ti qs_t e^{G_t - G_r}
    for (int ct = 2 * half; ct < 2 * half + 2; ++ct) {
        const int cc = 16 * ct + rr;
        f4 aE = {0, 0, 0, 0}, aQ = {0, 0, 0, 0}, aK = {0, 0, 0, 0};
        if (b > 0) {
            const int r = 16 * b;
            const float Gr = Gs[r * 64 + cc];
#pragma unroll 4
            for (int i0 = 0; i0 < r; i0 += 4) {
                const int i = i0 + gg;
                const float bv = Ks[i * 64 + cc] * ex2(Gr - Gs[i * 64 + cc]);
                aE = mfma_f32_k4(dMs[(r + rr) * C + i], bv, aE);
                aQ = mfma_f32_k4(dAqs[(r + rr) * C + i], bv, aQ);
            }
        }
        for (int b2 = b + 1; b2 < 4; ++b2) {
            const int r = 16 * b2;
            const float Gr = Gs[r * 64 + cc];
            f4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int k0 = 0; k0 < 16; k0 += 4) {
                const int t = r + k0 + gg;
                const float f = ex2(Gs[t * 64 + cc] - Gr);
                acc = mfma_f32_k4(dMs[t * C + 16 * b + rr], Es[t * 64 + cc] * f, acc);
                acc = mfma_f32_k4(dAqs[t * C + 16 * b + rr], Qs[t * 64 + cc] * f, acc);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int i = 16 * b + 4 * gg + s;
                aK[s] += acc[s] * ex2(Gs[r * 64 + 16 * ct + rr] - Gs[i * 64 + 16 * ct + rr]);
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int t = 16 * b + 4 * gg + s, ch = 16 * ct + rr;
            const float F = b > 0 ? ex2(Gs[t * 64 + ch] - Gs[16 * b * 64 + ch]) : 0.f;
            Te[t * 64 + ch] = aE[s] * F;
            Tq[t * 64 + ch] = aQ[s] * F;
            Ik[t * 64 + ch] = aK[s];
        }
    }
    __syncthreads();

    // pairs inside block b that the wave's rows take part in, lane = channel:
    // E = e^{G_t - G_i}, i <= t; as t the rows r0.., as i the same rows
    float sde[8], sdq[8], sdk[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
        const int t = r0 + x;
        sde[x] = Te[t * 64 + cl];
        sdq[x] = Tq[t * 64 + cl];
        sdk[x] = Ik[t * 64 + cl];
    }
    const int base = 16 * b;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
        const int tl = 8 * half + x, t = base + tl;
        const float Gt = Gs[t * 64 + cl];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int o = base + j;
            const float Go = Gs[o * 64 + cl];
            if (j <= tl) {  // o = i <= t: row t's sums
                const float E = ex2(Gt - Go), ko = Ks[o * 64 + cl];
                if (j < tl) sde[x] += dMs[t * C + o] * ko * E;
                sdq[x] += dAqs[t * C + o] * ko * E;
            }
            if (j >= tl) {  // o = t >= i with i = this row: row i's sum
                const float E = ex2(Go - Gt);
                float y = dAqs[o * C + t] * Qs[o * 64 + cl];
                if (j > tl) y += dMs[o * C + t] * Es[o * 64 + cl];
                sdk[x] += y * E;
            }
        }
    }

    // chain rule for the wave's rows
    const float GC = Gs[(C - 1) * 64 + cl];
    float dG[8], de[8], dq[8], dk[8], sKK = 0.f, bsum = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
        const int t = r0 + x;
        const float G = Gs[t * 64 + cl], eg = ex2(G), kg = ex2(GC - G);
        const float dEt = pdE[x], dQt = pdQ[x], dKh = pdK[x];
        const float e = Es[t * 64 + cl], qs = Qs[t * 64 + cl], kk = Ks[t * 64 + cl];
        const float te = sde[x], tq = sdq[x], ik = sdk[x];
        de[x] = eg * dEt + te;
        dq[x] = eg * dQt + tq;
        dk[x] = kg * dKh + ik;
        const float khv = kk * kg;
        dG[x] = dEt * (e * eg) + dQt * (qs * eg) - dKh * khv + e * te + qs * tq - kk * ik;
        sKK += dKh * khv;
        bsum += dG[x];
    }
    blk[w * 64 + cl] = bsum;
    gcp[w * 64 + cl] = sKK;
    __syncthreads();
    // dg_t = sum_{r >= t} dG_r; G_C (the last row) also enters through K-hat and gamma_C
    float carry = pgC * ex2(GC);
#pragma unroll
    for (int x = 0; x < NW; ++x) carry += gcp[x * 64 + cl];
    for (int x = w + 1; x < NW; ++x) carry += blk[x * 64 + cl];
    float alsum = 0.f;
#pragma unroll
    for (int x = 7; x >= 0; --x) {
        carry += dG[x];
        const int t = r0 + x;
        if (t < L) {
            const size_t ka = (((size_t)bb * p.T + t0 + t) * p.Hv + hv) * DK + c;
            const float av = bf16_to_f32(a[ka]), beta = sigmoid_fast(bf16_to_f32(er[ka]));
            const float kk = Ks[t * 64 + cl];
            const float dg = carry;  // natural-log units
            p.da[ka] = -dg * rate * sigmoid_fast(av);
            alsum += dg * (-rate * softplus_fast(av));
            p.derase[ka] = de[x] * kk * beta * (1.f - beta);
            ws.dqh[ka] = p.scale * dq[x];
            ws.dkh[ka] = dk[x] + de[x] * beta;
        }
    }
    alp[w * 64 + cl] = alsum;
    __syncthreads();
    if (w == 0) {
        float sa = 0.f;
#pragma unroll
        for (int x = 0; x < NW; ++x) sa += alp[x * 64 + cl];
        ws.dAl[(size_t)u * DK + c] = sa;
    }
    // dz = dR -> dv, d_write (the first channel group of each chunk)
    if (cg == 0) {
        const uint16_t *v = reinterpret_cast<const uint16_t *>(p.v), *wr = reinterpret_cast<const uint16_t *>(p.write);
        const float *dRu = ws.dR + (size_t)u * C * DV;
#pragma unroll
        for (int it = 0; it < C * DV / 8 / LOCAL_NT; ++it) {
            const int i = tid + LOCAL_NT * it, t = i / (DV / 8), j = (i % (DV / 8)) * 8, tl = min(t, L - 1);
            const size_t kv = (((size_t)bb * p.T + t0 + tl) * p.Hv + hv) * DV + j;
            f4 vv[2], om[2];
            bf8_to_f32(*reinterpret_cast<const u16x8 *>(v + kv), vv[0], vv[1]);
            bf8_to_f32(*reinterpret_cast<const u16x8 *>(wr + kv), om[0], om[1]);
            f4 dz[2] = {*reinterpret_cast<const f4 *>(dRu + t * DV + j), *reinterpret_cast<const f4 *>(dRu + t * DV + j + 4)};
            if (t < L) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    f4 o1, o2;
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const float sg = sigmoid_fast(om[hh][x]);
                        o1[x] = dz[hh][x] * sg;
                        o2[x] = dz[hh][x] * vv[hh][x] * sg * (1.f - sg);
                    }
                    *reinterpret_cast<f4 *>(p.dv + kv + 4 * hh) = o1;
                    *reinterpret_cast<f4 *>(p.dwrite + kv + 4 * hh) = o2;
                }
            }
        }
    }
}

// dq, dk: sums over the value heads of each key head; dA_log: sums over chunks.
template <int DK>
__global__ __launch_bounds__(256) void g2b_reduce(Bwd2Args p, Bwd2Workspace ws) {
    const int grp = p.Hv / p.Hk;
    const size_t nq = (size_t)p.B * p.T * p.Hk * DK;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < nq; i += (size_t)gridDim.x * 256) {
        const int c = i % DK;
        const size_t row = i / DK;  // (b, t, hk)
        const int hk = row % p.Hk;
        const size_t bt = row / p.Hk;
        float sq = 0.f, sk = 0.f;
        for (int x = 0; x < grp; ++x) {
            const size_t o = (bt * p.Hv + (size_t)hk * grp + x) * DK + c;
            sq += ws.dqh[o];
            sk += ws.dkh[o];
        }
        p.dq[i] = sq;
        p.dk[i] = sk;
    }
    const size_t na = (size_t)p.Hv * DK;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < na; i += (size_t)gridDim.x * 256) {
        const int hv = i / DK, c = i % DK;
        float s = 0.f;
        for (int bb = 0; bb < p.B; ++bb)
            for (int n = 0; n < p.NC; ++n) s += ws.dAl[unit_of(bb, hv, n, p.Hv, p.NC) * DK + c];
        p.dA_log[i] = s;
    }
}

// T = 0: dS0 = dS_T (or 0), dA_log = 0
__global__ void g2b_empty(float *dS0, const float *dST, size_t ns, float *dA_log, size_t na) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < ns + na; i += (size_t)gridDim.x * blockDim.x) {
        if (i < ns) {
            if (dS0) dS0[i] = dST ? dST[i] : 0.f;
        } else {
            dA_log[i - ns] = 0.f;
        }
    }
}

template <int DK, int DV>
hipError_t launch_bwd2_t(const Bwd2Args &p, const Bwd2Workspace &ws, hipStream_t s, const hipEvent_t *ev) {
    const unsigned units = (unsigned)(p.B * p.Hv * p.NC), slices = (unsigned)(p.B * p.Hv * (DV / 32));
    hipError_t e = hipSuccess;
    auto rec = [&](int i) {
        if (ev && e == hipSuccess) e = hipEventRecord(ev[i], s);
    };
    rec(0);
    hipLaunchKernelGGL((g2b_prep<DK, DV>), dim3(units), dim3(256), 0, s, p, ws);
    rec(1);
    hipLaunchKernelGGL((g2b_fwd_scan<DK, DV>), dim3(slices), dim3(256), 0, s, p, ws);
    rec(2);
    hipLaunchKernelGGL((g2b_bwd_scan<DK, DV>), dim3(slices), dim3(256), 0, s, p, ws);
    rec(3);
    hipLaunchKernelGGL((g2b_products<DK, DV>), dim3(units), dim3(256), 0, s, p, ws);
    rec(4);
    hipLaunchKernelGGL((g2b_local<DK, DV>), dim3(units * (DK / 64)), dim3(LOCAL_NT), 0, s, p, ws);
    rec(5);
    const size_t nq = (size_t)p.B * p.T * p.Hk * DK / 256 + 1;
    hipLaunchKernelGGL((g2b_reduce<DK>), dim3((unsigned)(nq < 65536 ? nq : 65536)), dim3(256), 0, s, p, ws);
    rec(6);
    const hipError_t le = hipGetLastError();
    return le != hipSuccess ? le : e;
}

}  // namespace

size_t bwd2_workspace_layout(int B, int T, int Hv, int Dk, int Dv, void *base, Bwd2Workspace *ws) {
    const size_t NC = ((size_t)T + C - 1) / C, U = (size_t)B * Hv * NC;
    size_t off = 0;
    auto take = [&](float **dst, size_t elems) {
        if (dst) *dst = base ? reinterpret_cast<float *>(static_cast<char *>(base) + off) : nullptr;
        off += (elems * 4 + 255) / 256 * 256;
    };
    Bwd2Workspace w{};
    take(&w.A, U * C * C);
    take(&w.Aq, U * C * C);
    take(&w.Et, U * C * Dk);
    take(&w.Qt, U * C * Dk);
    take(&w.Kh, U * C * Dk);
    take(&w.gC, U * Dk);
    take(&w.Z, U * C * Dv);
    take(&w.U, U * C * Dv);
    take(&w.R, U * C * Dv);
    take(&w.dU, U * C * Dv);
    take(&w.dR, U * C * Dv);
    take(&w.Sn, U * Dk * Dv);
    take(&w.dS1, U * Dk * Dv);
    take(&w.dEt, U * C * Dk);
    take(&w.dQt, U * C * Dk);
    take(&w.dKh, U * C * Dk);
    take(&w.dgC, U * Dk);
    take(&w.dM, U * C * C);
    take(&w.dAq, U * C * C);
    take(&w.dqh, (size_t)B * T * Hv * Dk);
    take(&w.dkh, (size_t)B * T * Hv * Dk);
    take(&w.dAl, U * Dk);
    w.bytes = off;
    if (ws) *ws = w;
    return off;
}

hipError_t launch_bwd2(const Bwd2Args &p, const Bwd2Workspace &ws, hipStream_t s, const hipEvent_t *ev) {
    if (p.B == 0) return hipSuccess;
    if (p.T == 0) {
        const size_t ns = (size_t)p.B * p.Hv * p.Dk * p.Dv, na = (size_t)p.Hv * p.Dk;
        hipLaunchKernelGGL(g2b_empty, dim3((unsigned)((ns + na) / 256 + 1 < 65536 ? (ns + na) / 256 + 1 : 65536)),
                           dim3(256), 0, s, p.dS0, p.dST, ns, p.dA_log, na);
        return hipGetLastError();
    }
    if (p.Dk == 128 && p.Dv == 128) return launch_bwd2_t<128, 128>(p, ws, s, ev);
    if (p.Dk == 128 && p.Dv == 64) return launch_bwd2_t<128, 64>(p, ws, s, ev);
    if (p.Dk == 64 && p.Dv == 128) return launch_bwd2_t<64, 128>(p, ws, s, ev);
    if (p.Dk == 64 && p.Dv == 64) return launch_bwd2_t<64, 64>(p, ws, s, ev);
    return hipErrorInvalidValue;
}

}  // namespace gdn
