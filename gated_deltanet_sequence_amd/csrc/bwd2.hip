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
// Every quantity is float32 (the inputs are bfloat16 or float32); the products of
// both scans and those over the value columns in g2b_products take their float32
// operands split into two bfloat16 halves (three bfloat16 matrix-core products per
// float32 product, about 2^-16 relative).  The work is split over six launches:
//   g2b_prep       per chunk: gates, images, M and Aq, A = (I + M)^{-1}
//   g2b_fwd_scan   per (sequence, head, 32 value columns): S_n, R, U over the chunks
//   g2b_bwd_scan   the same slices in reverse: dS_{n+1}, dU, dR; dS_0
//   g2b_products   per chunk: dEt, dQt, dKh, dgamma_C, dAq, dM
//   g2b_local      per (chunk, 32 key channels): pairwise decay sums, gate chain
//   g2b_reduce     dq, dk over the value heads of a key head; dA_log over chunks
// Decay factors never exceed 1: a product e^{G_t - G_i} over a 16-token block
// pair below the diagonal is split at the block's first row r (i < r <= t) into
// e^{G_t - G_r} e^{G_r - G_i}; inside a diagonal block it is either taken
// directly or split at dyadic sub-blocks (first token of the second half).
#include <type_traits>

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

// 8 consecutive input elements (bfloat16 or float32) held in registers between
// their load and their conversion to float32.
template <typename TIn> struct In8;
template <> struct In8<bf16_t> {
    u16x8 x;
    __device__ __forceinline__ void load(const bf16_t *p, size_t i) {
        x = *reinterpret_cast<const u16x8 *>(reinterpret_cast<const uint16_t *>(p) + i);
    }
    __device__ __forceinline__ void get(f4 &lo, f4 &hi) const { bf8_to_f32(x, lo, hi); }
};
template <> struct In8<float> {
    f4 lo_, hi_;
    __device__ __forceinline__ void load(const float *p, size_t i) {
        lo_ = *reinterpret_cast<const f4 *>(p + i);
        hi_ = *reinterpret_cast<const f4 *>(p + i + 4);
    }
    __device__ __forceinline__ void get(f4 &lo, f4 &hi) const {
        lo = lo_;
        hi = hi_;
    }
};

// 4 consecutive input elements held raw in registers between their load and
// their conversion to float32 (so that a phase can issue all its loads first).
template <typename TIn> struct In4;
template <> struct In4<bf16_t> {
    u16x4 x;
    __device__ __forceinline__ void load(const bf16_t *p, size_t i) {
        x = *reinterpret_cast<const u16x4 *>(reinterpret_cast<const uint16_t *>(p) + i);
    }
    __device__ __forceinline__ f4 get() const {
        return f4{bf16_to_f32(x[0]), bf16_to_f32(x[1]), bf16_to_f32(x[2]), bf16_to_f32(x[3])};
    }
};
template <> struct In4<float> {
    f4 x;
    __device__ __forceinline__ void load(const float *p, size_t i) { x = *reinterpret_cast<const f4 *>(p + i); }
    __device__ __forceinline__ f4 get() const { return x; }
};

// One input element held raw in registers between its load and its use.
template <typename TIn> struct In1;
template <> struct In1<bf16_t> {
    uint16_t x;
    __device__ __forceinline__ void load(const bf16_t *p, size_t i) { x = reinterpret_cast<const uint16_t *>(p)[i]; }
    __device__ __forceinline__ float get() const { return bf16_to_f32(x); }
};
template <> struct In1<float> {
    float x;
    __device__ __forceinline__ void load(const float *p, size_t i) { x = p[i]; }
    __device__ __forceinline__ float get() const { return x; }
};

// A ROWS x COLS float32 tile (row-major, source rows SS floats apart) held in
// registers between its global load and its LDS store: the scans load the next
// chunk's operands while computing the current one.
template <int ROWS, int COLS, int NT = 256, int SS = COLS> struct RegTile {
    static constexpr int PER = ROWS * COLS / 4 / NT;
    static_assert(ROWS * COLS / 4 % NT == 0, "tile size");
    f4 x[PER];
    __device__ __forceinline__ void load(const float *__restrict__ src) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int i = threadIdx.x + j * NT, r = i / (COLS / 4), c = (i % (COLS / 4)) * 4;
            x[j] = *reinterpret_cast<const f4 *>(src + (size_t)r * SS + c);
        }
    }
    template <int LS> __device__ __forceinline__ void store(float *dst, float f = 1.f) const {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int i = threadIdx.x + j * NT, r = i / (COLS / 4), c = (i % (COLS / 4)) * 4;
            *reinterpret_cast<f4 *>(dst + r * LS + c) = x[j] * f;
        }
    }
};

// work-group barrier for hand-offs through LDS only: each wave's LDS accesses
// complete before it (lgkmcnt(0)), while its global loads and stores stay in
// flight (no launch here passes data between waves through global memory).
// Measured against __syncthreads() in the same places: no difference in time.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 2^x on the hardware unit (arguments here are <= 0: every decay factor is at most 1)
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ size_t unit_of(int bb, int hv, int n, int Hv, int NC) {
    return ((size_t)bb * Hv + hv) * NC + n;
}

// ---------------------------------------------------------------------------
// g2b_prep: one work-group of 8 waves per (sequence, value head, chunk).  The
// key channels are taken 64 at a time (M, Aq and the diagonal of Aq are sums
// over them, accumulated across the halves), so that the tiles take 78 KB of
// LDS and two work-groups share a CU (four waves per SIMD); waves 0..3 take the
// diagonal tiles of M and Aq while waves 4..7 take those below the diagonal.
// ---------------------------------------------------------------------------
constexpr int PREP_NT = 512;

template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(PREP_NT, 4) void g2b_prep(Bwd2Args p, Bwd2Workspace ws) {
    constexpr int DH = 64, NH = DK / DH;  // channels per pass, passes
    constexpr int LS = DH + 4;            // conflict-free for lanes (row = l%16, col = l/16)
    __shared__ __attribute__((aligned(16))) float sm[4 * C * LS + C];
    float *Gs = sm, *Es = Gs + C * LS, *Qs = Es + C * LS, *Ks = Qs + C * LS, *dd = Ks + C * LS;
    float *Ms = Es, *As = Qs, *Xt = Ks;  // after the tiles: M, A (stride 68), 4 x [16][48] scratch
    static_assert(LS == 68 && C * LS >= 4 * 16 * 48, "M, A and the scratch reuse the tile space");

    const int u = blockIdx.x, NC = p.NC;
    const int n = u % NC, hv = (u / NC) % p.Hv, bb = u / (NC * p.Hv), hk = hv / (p.Hv / p.Hk);
    const int t0 = n * C, L = min(C, p.T - t0);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, rr = lane & 15, gg = lane >> 4;

    // 1. gates: G (log2 units, 0 past T), e = sigmoid(erase) k, qs = scale q, k (z = sigmoid(write) v
    //    is formed by the forward scan from the inputs).
    //    Thread = (4 channels of the pass, a group of RPT consecutive rows); rows past T read
    //    the last token (L >= 1) and are zeroed, so every load is unconditional.  The in-chunk
    //    prefix of g is taken over the thread's rows, then the totals of the earlier row
    //    groups are added.  Both passes' loads are issued before any is used.
    constexpr int NQ = DH / 4, NRG = PREP_NT / NQ, RPT = C / NRG;
    __shared__ float tot[NRG * DH];
    const int cq = (tid % NQ) * 4, rg = tid / NQ;
    In4<TIn> rk[NH][RPT], rq[NH][RPT], ra[NH][RPT], re[NH][RPT];
    f4 al[NH];
    {
        const TIn *qb = static_cast<const TIn *>(p.q), *kb = static_cast<const TIn *>(p.k);
        const TIn *ab = static_cast<const TIn *>(p.a), *eb = static_cast<const TIn *>(p.erase);
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const int c = DH * h + cq;
            al[h] = *reinterpret_cast<const f4 *>(p.A_log + (size_t)hv * DK + c);
#pragma unroll
            for (int x = 0; x < RPT; ++x) {
                const int tl = min(rg * RPT + x, L - 1);
                const size_t kq = (((size_t)bb * p.T + t0 + tl) * p.Hk + hk) * DK + c;
                const size_t ka = (((size_t)bb * p.T + t0 + tl) * p.Hv + hv) * DK + c;
                rk[h][x].load(kb, kq);
                rq[h][x].load(qb, kq);
                ra[h][x].load(ab, ka);
                re[h][x].load(eb, ka);
            }
        }
    }
    // tile ti = 0..5 below the diagonal, row by row: (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
    // (computed: a constexpr table was placed in global memory and loaded per use)
    auto obt = [](int ti) { return ti < 1 ? 1 : ti < 3 ? 2 : 3; };
    auto obi = [&](int ti) { const int bt = obt(ti); return ti - bt * (bt - 1) / 2; };
    f4 mO[2], qO[2], mD = {0, 0, 0, 0}, qD = {0, 0, 0, 0};
#pragma unroll
    for (int x = 0; x < 2; ++x) mO[x] = qO[x] = f4{0, 0, 0, 0};
    float ddacc = 0.f;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        if (h > 0) __syncthreads();  // the previous pass is done with the tiles
        {
            f4 rate;
#pragma unroll
            for (int j = 0; j < 4; ++j) rate[j] = -exp_fast(al[h][j]) * LOG2E;
            f4 run = {0, 0, 0, 0}, gr[RPT];
#pragma unroll
            for (int x = 0; x < RPT; ++x) {
                const int t = rg * RPT + x;
                const f4 kk = rk[h][x].get(), qq = rq[h][x].get(), aa = ra[h][x].get(), ee = re[h][x].get();
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
                *reinterpret_cast<f4 *>(Es + t * LS + cq) = ev;
                *reinterpret_cast<f4 *>(Qs + t * LS + cq) = qv;
                *reinterpret_cast<f4 *>(Ks + t * LS + cq) = kv;
            }
            *reinterpret_cast<f4 *>(tot + rg * DH + cq) = run;
            __syncthreads();
            f4 off = {0, 0, 0, 0};
            for (int x = 0; x < rg; ++x) off += *reinterpret_cast<const f4 *>(tot + x * DH + cq);
#pragma unroll
            for (int x = 0; x < RPT; ++x) *reinterpret_cast<f4 *>(Gs + (rg * RPT + x) * LS + cq) = gr[x] + off;
        }
        __syncthreads();
        // 3. images, gamma_C and the diagonal of Aq (q_t . k_t, no decay) for the pass's channels
        {
            const size_t ub = (size_t)u * C * DK + DH * h;
            for (int i = tid; i < C * DH / 4; i += PREP_NT) {
                const int t = i / (DH / 4), c = (i % (DH / 4)) * 4;
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
            for (int c = tid; c < DH; c += PREP_NT) ws.gC[(size_t)u * DK + DH * h + c] = ex2(Gs[(C - 1) * LS + c]);
            if (tid < C) {
#pragma unroll 8
                for (int c = 0; c < DH; ++c) ddacc += Qs[tid * LS + c] * Ks[tid * LS + c];
            }
        }
        // 4. M and Aq over the pass's channels.  Tiles below the diagonal (bt > bi),
        //    reference row r = 16 bt: sum_c [e_t e^{G_t - G_r}] [k_i e^{G_r - G_i}].  Waves
        //    4..7 take tiles w - 4 and w (while waves 0..3 take the diagonal tiles).
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int ti = w - 4 + 4 * x;
            if (w >= 4 && ti < 6) {
                const int bt = obt(ti), bi = obi(ti), r = 16 * bt, t = 16 * bt + rr, i = 16 * bi + rr;
#pragma unroll 8
                for (int c0 = 0; c0 < DH; c0 += 4) {
                    const int c = c0 + gg;
                    const float Gr = Gs[r * LS + c];
                    const float ft = ex2(Gs[t * LS + c] - Gr), b = Ks[i * LS + c] * ex2(Gr - Gs[i * LS + c]);
                    mO[x] = mfma_f32_k4(Es[t * LS + c] * ft, b, mO[x]);
                    qO[x] = mfma_f32_k4(Qs[t * LS + c] * ft, b, qO[x]);
                }
            }
        }
        //    Diagonal tile w (waves 0..3): dyadic levels (half sizes 8, 4, 2, 1); a pair
        //    (t > i) of the tile belongs to the level whose 2h-block holds both with i in
        //    the first and t in the second half; reference = first token of that half.
        if (w < 4) {
            const int base = 16 * w, t = base + rr, i = base + rr;
#pragma unroll
            for (int hl = 8; hl >= 1; hl >>= 1) {
                const bool tsec = (rr & hl) != 0;
                const int rt = base + (rr & ~(hl - 1)), ri = base + ((rr | hl) & ~(hl - 1));
                f4 aM = {0, 0, 0, 0}, aQ = {0, 0, 0, 0};
#pragma unroll 8
                for (int c0 = 0; c0 < DH; c0 += 4) {
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
                    if (((tl ^ rr) & ~(2 * hl - 1)) == 0 && (tl & hl) && !(rr & hl)) {
                        mD[s] += aM[s];
                        qD[s] += aQ[s];
                    }
                }
            }
        }
    }
    if (tid < C) dd[tid] = ddacc;
    __syncthreads();  // Es, Qs, Ks are reused below; dd complete
    if (w < 4) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            if (4 * gg + s == rr) qD[s] += dd[16 * w + rr];
    }
    // Aq to the workspace (zero above the diagonal); M into LDS (zero on and above)
    {
        float *Aqu = ws.Aq + (size_t)u * C * C;
        for (int i = tid; i < C * 68; i += PREP_NT) Ms[i] = 0.f;
        __syncthreads();
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int ti = w - 4 + 4 * x;
            if (w >= 4 && ti < 6) {
                const int bt = obt(ti), bi = obi(ti);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int t = 16 * bt + 4 * gg + s, i = 16 * bi + rr;
                    Ms[t * 68 + i] = mO[x][s];
                    Aqu[t * C + i] = qO[x][s];
                    Aqu[i * C + t] = 0.f;  // the mirrored tile above the diagonal
                }
            }
        }
        if (w < 4) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int t = 16 * w + 4 * gg + s, i = 16 * w + rr;
                Ms[t * 68 + i] = mD[s];
                Aqu[t * C + i] = qD[s];
            }
        }
    }
    __syncthreads();
    // 5. A = (I + M)^{-1}: diagonal 16 x 16 blocks by forward substitution (wave w,
    //    lane j < 16 owns column j of block w), then block rows 1..3:
    //    A_bj = -A_bb sum_{m=j}^{b-1} M_bm A_mj.
    if (w < 4 && lane < 16) {
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
    for (int i = tid; i < C * C; i += PREP_NT) {
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
    for (int i = tid; i < C * C / 4; i += PREP_NT) {
        const int t = i / (C / 4), c = (i % (C / 4)) * 4;
        *reinterpret_cast<f4 *>(Au + t * C + c) = *reinterpret_cast<const f4 *>(As + t * 68 + c);
    }
}

// ---------------------------------------------------------------------------
// Split-bfloat16 products.  A float32 x is held as hi = bf16(x) and
// lo = bf16(x - hi) (round to nearest even both times), so that x = hi + lo to
// about 2^-17 relative; a product x y is then formed as hi_x hi_y + hi_x lo_y +
// lo_x hi_y on the 16x16x32 bfloat16 matrix cores with a float32 accumulator
// (the dropped lo_x lo_y is below 2^-16 |x y|): three 32-deep products in place
// of eight 4-deep float32 ones.
// ---------------------------------------------------------------------------
typedef __bf16 bf8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f4 mfma_bf16_k32(bf8v a, bf8v b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 4 float32 values to their hi and lo halves (8 bytes each)
__device__ __forceinline__ void split4(f4 x, u16x4 &hi, u16x4 &lo) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const __bf16 h = (__bf16)x[j];
        hi[j] = __builtin_bit_cast(uint16_t, h);
        lo[j] = __builtin_bit_cast(uint16_t, (__bf16)(x[j] - (float)h));
    }
}

// acc += A(16 x K) B(K x 16), A(m, k) at ah/al[m * LA + k], B(k, n) at bh/bl[n * LB + k]
// (both contraction-contiguous, split halves in LDS).  Lane l supplies row / column l%16,
// contraction elements 8 (l/16) .. 8 (l/16) + 7 of each 32-deep step.  ALO = false: A is
// exact in bfloat16 (its lo half is zero and is not read).
template <int K, int LA, int LB, bool ALO>
__device__ __forceinline__ void mma_x3(f4 &acc, const uint16_t *ah, const uint16_t *al, const uint16_t *bh,
                                       const uint16_t *bl) {
    const int l = threadIdx.x & 63, r = l & 15, g = l >> 4;
    const int oa = r * LA + 8 * g, ob = r * LB + 8 * g;
#pragma unroll
    for (int k = 0; k < K; k += 32) {
        const bf8v a_h = *reinterpret_cast<const bf8v *>(ah + oa + k);
        const bf8v b_h = *reinterpret_cast<const bf8v *>(bh + ob + k);
        const bf8v b_l = *reinterpret_cast<const bf8v *>(bl + ob + k);
        if constexpr (ALO) acc = mfma_bf16_k32(*reinterpret_cast<const bf8v *>(al + oa + k), b_h, acc);
        acc = mfma_bf16_k32(a_h, b_l, acc);
        acc = mfma_bf16_k32(a_h, b_h, acc);
    }
}

// A ROWS x COLS float32 register tile (see RegTile) stored split: rows of stride LS
template <int ROWS, int COLS, int LS, int SS = COLS, int NT = 256>
__device__ __forceinline__ void store_split(const RegTile<ROWS, COLS, NT, SS> &t, uint16_t *hi, uint16_t *lo,
                                            float f = 1.f) {
#pragma unroll
    for (int j = 0; j < RegTile<ROWS, COLS, NT, SS>::PER; ++j) {
        const int i = threadIdx.x + j * NT, r = i / (COLS / 4), c = (i % (COLS / 4)) * 4;
        u16x4 h, l;
        split4(t.x[j] * f, h, l);
        *reinterpret_cast<u16x4 *>(hi + r * LS + c) = h;
        *reinterpret_cast<u16x4 *>(lo + r * LS + c) = l;
    }
}

// k-block operands of one 32-deep split product (see the MFMA layouts in
// gdn_device.h): lane (g, r) = (l/16, l%16) holds, for the two 16-deep blocks
// kb0, kb0 + 1 of the step, the 4 values k = 16 kb + 4 g + 0..3 of row / column r
// -- the rows an accumulator tile holds, so accumulator tiles are operands as
// they are.
typedef short s4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4v lds_s4v;
struct KOp {
    u16x4 h0, h1, l0, l1;
};
__device__ __forceinline__ bf8v cat8(u16x4 a, u16x4 b) {
    return __builtin_bit_cast(bf8v, u16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]});
}
// acc += A B over one 32-deep step; ALO / BLO: the operand has a lo half
template <bool ALO, bool BLO>
__device__ __forceinline__ f4 x3_step(f4 acc, const KOp &a, const KOp &b) {
    const bf8v ah = cat8(a.h0, a.h1), bh = cat8(b.h0, b.h1);
    if constexpr (ALO) acc = mfma_bf16_k32(cat8(a.l0, a.l1), bh, acc);
    if constexpr (BLO) acc = mfma_bf16_k32(ah, cat8(b.l0, b.l1), acc);
    return mfma_bf16_k32(ah, bh, acc);
}
// from a split tile X[m][k] with k contiguous (row stride S): row m0 + r
template <int S, bool LO>
__device__ __forceinline__ KOp op_row(const uint16_t *h, const uint16_t *l, int m0, int kb0) {
    const int ln = threadIdx.x & 63, o = (m0 + (ln & 15)) * S + 16 * kb0 + 4 * (ln >> 4);
    KOp x;
    x.h0 = *reinterpret_cast<const u16x4 *>(h + o);
    x.h1 = *reinterpret_cast<const u16x4 *>(h + o + 16);
    if constexpr (LO) {
        x.l0 = *reinterpret_cast<const u16x4 *>(l + o);
        x.l1 = *reinterpret_cast<const u16x4 *>(l + o + 16);
    }
    return x;
}
// from a split tile T[k][m] with m contiguous (row stride S), read transposed
// (ds_read_b64_tr_b16: in each 16-lane group, lane 4i + q points at 4 values,
// columns 4q .. 4q+3 of row i of a 4 x 16 block, and lane j receives column j of
// the 4 rows): column m0 + r
__device__ __forceinline__ u16x4 lds_tr4(const uint16_t *p) {
    return __builtin_bit_cast(u16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v *)p));
}
template <int S, bool LO>
__device__ __forceinline__ KOp op_tr(const uint16_t *h, const uint16_t *l, int m0, int kb0) {
    const int ln = threadIdx.x & 63, r = ln & 15;
    const int o = (16 * kb0 + 4 * (ln >> 4) + (r >> 2)) * S + m0 + 4 * (r & 3);
    KOp x;
    x.h0 = lds_tr4(h + o);
    x.h1 = lds_tr4(h + o + 16 * S);
    if constexpr (LO) {
        x.l0 = lds_tr4(l + o);
        x.l1 = lds_tr4(l + o + 16 * S);
    }
    return x;
}
// an accumulator tile (rows 16 kb + 4 g + s, column 16 jb + r) into a split
// transposed store XT[n][k] (row stride S): 8 bytes per half and lane
template <int S>
__device__ __forceinline__ void store_acc_t(f4 x, uint16_t *h, uint16_t *l, int kb, int jb) {
    const int ln = threadIdx.x & 63, o = (16 * jb + (ln & 15)) * S + 16 * kb + 4 * (ln >> 4);
    u16x4 xh, xl;
    split4(x, xh, xl);
    *reinterpret_cast<u16x4 *>(h + o) = xh;
    *reinterpret_cast<u16x4 *>(l + o) = xl;
}

// ROWS x COLS float32 block (row-major, contiguous) into split LDS rows of stride LS,
// times f; loads in batches of 8 per thread as lds_load.
template <int ROWS, int COLS, int LS, int NT = 256>
__device__ __forceinline__ void lds_load_split(uint16_t *hi, uint16_t *lo, const float *__restrict__ src, float f = 1.f) {
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
            u16x4 h, l;
            split4(x[j] * f, h, l);
            *reinterpret_cast<u16x4 *>(hi + r * LS + c) = h;
            *reinterpret_cast<u16x4 *>(lo + r * LS + c) = l;
        }
    }
}

// ---------------------------------------------------------------------------
// g2b_fwd_scan: one work-group of 8 waves per (sequence, value head, 32 value
// columns) (two waves per SIMD: one alone left every latency of the chunk's
// dependent products exposed); wave w holds state tiles as MFMA accumulators
// and the R, U tile (row block w % 4, column block w / 4).
// Its products take split operands.  LDS (16-bit elements, each split tile a
// hi and a lo array): Et, Kh [C][DK], A [C][C], and the transposed S [32][DK],
// R, U [32][C] of the chunk.
// ---------------------------------------------------------------------------
template <int DK> struct FwdScanLds {
    static constexpr int SK = DK + 8, SA = C + 8, SS = DK + 8, SU = C + 8;
    static constexpr int E_ = 0, K_ = E_ + 2 * C * SK, A_ = K_ + 2 * C * SK, S_ = A_ + 2 * C * SA,
                         R_ = S_ + 2 * 32 * SS, U_ = R_ + 2 * 32 * SU, END = U_ + 2 * 32 * SU;
};

constexpr int SCAN_NT = 512;

// work-group -> (head = sequence * H_v + value head, column slice): work-group i runs on
// XCD i % 8, so heads go eight at a time across the XCDs with the slices of each
// (which read the same per-chunk tiles) on one of them
__device__ __forceinline__ void scan_slice(int heads, int ns, int &head, int &js) {
    const int full = heads / 8 * 8 * ns, i = (int)blockIdx.x;
    if (i < full) {
        const int j = i / 8;
        head = 8 * (j / ns) + i % 8;
        js = j % ns;
    } else {
        head = heads / 8 * 8 + (i - full) / ns;
        js = (i - full) % ns;
    }
}

template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(SCAN_NT) void g2b_fwd_scan(Bwd2Args p, Bwd2Workspace ws) {
    typedef FwdScanLds<DK> FL;
    constexpr int SK = FL::SK, SA = FL::SA, SS = FL::SS, SU = FL::SU, NS = DV / 32, NT = DK / 16 * 2 / (SCAN_NT / 64);
    __shared__ __attribute__((aligned(16))) uint16_t lds[FL::END];
    uint16_t *EH = lds + FL::E_, *EL = EH + C * SK, *KH = lds + FL::K_, *KL = KH + C * SK, *AH = lds + FL::A_,
             *AL = AH + C * SA, *SH = lds + FL::S_, *SL = SH + 32 * SS, *RH = lds + FL::R_, *RL = RH + 32 * SU,
             *UH = lds + FL::U_, *UL = UH + 32 * SU;
    int head, js;
    scan_slice(p.B * p.Hv, NS, head, js);
    const int hv = head % p.Hv, bb = head / p.Hv, j0 = 32 * js;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, rr = lane & 15, gg = lane >> 4, NC = p.NC;
    const int rb = w & 3, ob = w >> 2;  // the wave's R, U tile: row block, column block
    // initial state: every load issued before any is used (one wait, not one per element)
    f4 S[NT];
    if (p.S0) {
#pragma unroll
        for (int x = 0; x < NT; ++x) {
            const int id = w * NT + x, cb = id >> 1, jb = id & 1;
#pragma unroll
            for (int s = 0; s < 4; ++s)
                S[x][s] = p.S0[(((size_t)bb * p.Hv + hv) * DK + 16 * cb + 4 * gg + s) * DV + j0 + 16 * jb + rr];
        }
    } else {
#pragma unroll
        for (int x = 0; x < NT; ++x) S[x] = f4{0, 0, 0, 0};
    }
#pragma unroll
    for (int x = 0; x < NT; ++x) {
        const int id = w * NT + x;
        store_acc_t<SS>(S[x], SH, SL, id >> 1, id & 1);
    }
    // this lane's v and write-logit elements of chunk m (rows past T read the last
    // token and are zeroed at use): loaded one chunk ahead, raw, for z = sigmoid(write) v
    const TIn *vin = static_cast<const TIn *>(p.v), *win = static_cast<const TIn *>(p.write);
    In1<TIn> zv[4], zw[4];
    auto load_z = [&](int m) {
        const int tm = m * C, Lm = min(C, p.T - tm);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int t = min(16 * rb + 4 * gg + s, Lm - 1);
            const size_t kv = (((size_t)bb * p.T + tm + t) * p.Hv + hv) * DV + j0 + 16 * ob + rr;
            zv[s].load(vin, kv);
            zw[s].load(win, kv);
        }
    };
    // the chunk's Et, Kh, A tiles: loaded a whole chunk ahead, into registers
    RegTile<C, DK, SCAN_NT> tE, tK;
    RegTile<C, C, SCAN_NT> tA;
    auto load_tiles = [&](int m) {
        const size_t um = unit_of(bb, hv, m, p.Hv, NC);
        tE.load(ws.Et + um * C * DK);
        tK.load(ws.Kh + um * C * DK);
        tA.load(ws.A + um * C * C);
    };
    if (NC > 0) {
        load_z(0);
        load_tiles(0);
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
        const float *gCu = ws.gC + u * DK;
        const int L = min(C, p.T - n * C);
        float zr[4], gcr[NT][4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
            zr[s] = zv[s].get() * sigmoid_fast(zw[s].get()) * (16 * rb + 4 * gg + s < L ? 1.f : 0.f);
#pragma unroll
        for (int x = 0; x < NT; ++x)
#pragma unroll
            for (int s = 0; s < 4; ++s) gcr[x][s] = gCu[16 * ((w * NT + x) >> 1) + 4 * gg + s];
        store_split<C, DK, SK>(tE, EH, EL);
        store_split<C, DK, SK>(tK, KH, KL);
        store_split<C, C, SA>(tA, AH, AL);
        // the next chunk's inputs, in flight during this chunk's products.  Issued on
        // every chunk (the last one reloads itself, unused): behind a branch, the paths
        // joined with different loads in flight and the compiler's wait at the join, for a
        // value loaded before them, became a wait for every load, the prefetch included.
        {
            const int nn = min(n + 1, NC - 1);
            load_z(nn);
            load_tiles(nn);
        }
        lds_barrier();
        // R = Z - Et S (the wave's tile)
        float *Ru = ws.R + u * C * DV, *Uu = ws.U + u * C * DV;
        {
            f4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < DK / 16; kb += 2)
                acc = x3_step<true, true>(acc, op_row<SK, true>(EH, EL, 16 * rb, kb), op_row<SS, true>(SH, SL, 16 * ob, kb));
            f4 rv;
#pragma unroll
            for (int s = 0; s < 4; ++s) rv[s] = zr[s] - acc[s];
            store_acc_t<SU>(rv, RH, RL, rb, ob);
#pragma unroll
            for (int s = 0; s < 4; ++s) Ru[(16 * rb + 4 * gg + s) * DV + j0 + 16 * ob + rr] = rv[s];
        }
        lds_barrier();
        // U = A R
        {
            f4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < C / 16; kb += 2)
                acc = x3_step<true, true>(acc, op_row<SA, true>(AH, AL, 16 * rb, kb), op_row<SU, true>(RH, RL, 16 * ob, kb));
            store_acc_t<SU>(acc, UH, UL, rb, ob);
#pragma unroll
            for (int s = 0; s < 4; ++s) Uu[(16 * rb + 4 * gg + s) * DV + j0 + 16 * ob + rr] = acc[s];
        }
        lds_barrier();
        // S = gamma_C . S + Kh^T U
#pragma unroll
        for (int x = 0; x < NT; ++x) {
            const int id = w * NT + x, cb = id >> 1, jb = id & 1;
#pragma unroll
            for (int s = 0; s < 4; ++s) S[x][s] *= gcr[x][s];
#pragma unroll
            for (int kb = 0; kb < C / 16; kb += 2)
                S[x] = x3_step<true, true>(S[x], op_tr<SK, true>(KH, KL, 16 * cb, kb), op_row<SU, true>(UH, UL, 16 * jb, kb));
            store_acc_t<SS>(S[x], SH, SL, cb, jb);
        }
        lds_barrier();
    }
}

// ---------------------------------------------------------------------------
// g2b_bwd_scan: the same slices and waves, chunks in reverse; dS in MFMA
// accumulators, the wave's dU, dR tile as in the forward scan.
// ---------------------------------------------------------------------------
// The reverse scan's products take split operands.  Its LDS (16-bit elements,
// each split tile a hi and a lo array):
// A_qk then A [C][C]; Kh then -Et [C][DK]; Qt [C][DK]; dO [C][32]; and the
// transposed dS [32][DK], dU, dR [32][C] of the chunk.
template <int DK> struct BwdScanLds {
    static constexpr int SA = C + 8, SK = DK + 8, SO = 32 + 8, SS = DK + 8, SU = C + 8;
    static constexpr int A_ = 0, K1_ = A_ + 2 * C * SA, K2_ = K1_ + 2 * C * SK, O_ = K2_ + 2 * C * SK,
                         S_ = O_ + 2 * C * SO, U_ = S_ + 2 * 32 * SS, R_ = U_ + 2 * 32 * SU, END = R_ + 2 * 32 * SU;
};

template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(SCAN_NT) void g2b_bwd_scan(Bwd2Args p, Bwd2Workspace ws) {
    typedef BwdScanLds<DK> BL;
    constexpr int SA = BL::SA, SK = BL::SK, SO = BL::SO, SS = BL::SS, SU = BL::SU;
    constexpr int NS = DV / 32, NT = DK / 16 * 2 / (SCAN_NT / 64);
    constexpr bool DO_LO = !std::is_same<TIn, bf16_t>::value;  // dO is exact in bfloat16 for bf16 inputs
    __shared__ __attribute__((aligned(16))) uint16_t lds[BL::END];
    uint16_t *AH = lds + BL::A_, *AL = AH + C * SA, *K1H = lds + BL::K1_, *K1L = K1H + C * SK;
    uint16_t *K2H = lds + BL::K2_, *K2L = K2H + C * SK, *OH = lds + BL::O_, *OL = OH + C * SO;
    uint16_t *DSH = lds + BL::S_, *DSL = DSH + 32 * SS, *DUH = lds + BL::U_, *DUL = DUH + 32 * SU;
    uint16_t *DRH = lds + BL::R_, *DRL = DRH + 32 * SU;
    int head, js;
    scan_slice(p.B * p.Hv, NS, head, js);
    const int hv = head % p.Hv, bb = head / p.Hv, j0 = 32 * js;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, rr = lane & 15, gg = lane >> 4, NC = p.NC;
    const int rb = w & 3, ob = w >> 2;  // the wave's dU, dR tile: row block, column block
    const TIn *dout = static_cast<const TIn *>(p.dout);
    // gradient of the final state: every load issued before any is used.  Wave w
    // holds the tiles (channel block cb, column block jb) id = w NT + x, cb = id / 2.
    f4 dS[NT];
    if (p.dST) {
#pragma unroll
        for (int x = 0; x < NT; ++x) {
            const int id = w * NT + x, cb = id >> 1, jb = id & 1;
#pragma unroll
            for (int s = 0; s < 4; ++s)
                dS[x][s] = p.dST[(((size_t)bb * p.Hv + hv) * DK + 16 * cb + 4 * gg + s) * DV + j0 + 16 * jb + rr];
        }
    } else {
#pragma unroll
        for (int x = 0; x < NT; ++x) dS[x] = f4{0, 0, 0, 0};
    }
#pragma unroll
    for (int x = 0; x < NT; ++x) {
        const int id = w * NT + x;
        store_acc_t<SS>(dS[x], DSH, DSL, id >> 1, id & 1);
    }
    // dO slice of chunk n: 64 rows x 32 columns, 8 per thread of the first 256 (rows past T
    // read the last token and are zeroed when stored)
    const int ot = (tid & 255) >> 2, oj = (tid & 3) * 8;
    const bool dot = tid < 256;
    auto load_do = [&](int n) {
        const int L = min(C, p.T - n * C), tl = min(ot, L - 1);
        In8<TIn> x;
        if (dot) x.load(dout, (((size_t)bb * p.T + n * C + tl) * p.Hv + hv) * DV + j0 + oj);
        return x;
    };
    auto store_do = [&](const In8<TIn> &x, int n) {
        if (!dot) return;
        const int L = min(C, p.T - n * C);
        f4 lo, hi;
        x.get(lo, hi);
        const float on = ot < L ? 1.f : 0.f;
        u16x4 h0, l0, h1, l1;
        split4(lo * on, h0, l0);
        split4(hi * on, h1, l1);
        *reinterpret_cast<u16x8 *>(OH + ot * SO + oj) = u16x8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
        if constexpr (DO_LO)
            *reinterpret_cast<u16x8 *>(OL + ot * SO + oj) = u16x8{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
    };
    // staged for the chunk about to run: A_qk, Kh, dO
    RegTile<C, C, SCAN_NT> rAq, rA;
    RegTile<C, DK, SCAN_NT> rKh, rQ, rE;
    In8<TIn> rdo;
    {
        const size_t u = unit_of(bb, hv, NC - 1, p.Hv, NC);
        rAq.load(ws.Aq + u * C * C);
        rKh.load(ws.Kh + u * C * DK);
        rdo = load_do(NC - 1);
        store_split<C, C, SA>(rAq, AH, AL);
        store_split<C, DK, SK>(rKh, K1H, K1L);
        store_do(rdo, NC - 1);
        rA.load(ws.A + u * C * C);
        rQ.load(ws.Qt + u * C * DK);
        rE.load(ws.Et + u * C * DK);
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
        lds_barrier();
        // dU = Aq^T dO + Kh dS  (the wave's tile)
        float *dUu = ws.dU + u * C * DV, *dRu = ws.dR + u * C * DV;
        {
            f4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < C / 16; kb += 2)
                acc = x3_step<true, DO_LO>(acc, op_tr<SA, true>(AH, AL, 16 * rb, kb), op_tr<SO, DO_LO>(OH, OL, 16 * ob, kb));
#pragma unroll
            for (int kb = 0; kb < DK / 16; kb += 2)
                acc = x3_step<true, true>(acc, op_row<SK, true>(K1H, K1L, 16 * rb, kb), op_row<SS, true>(DSH, DSL, 16 * ob, kb));
            store_acc_t<SU>(acc, DUH, DUL, rb, ob);
#pragma unroll
            for (int s = 0; s < 4; ++s) dUu[(16 * rb + 4 * gg + s) * DV + j0 + 16 * ob + rr] = acc[s];
        }
        lds_barrier();
        store_split<C, C, SA>(rA, AH, AL);
        store_split<C, DK, SK>(rQ, K2H, K2L);
        store_split<C, DK, SK>(rE, K1H, K1L, -1.f);
        // the next chunk's tiles in flight while this one finishes (A, Qt, Et a whole
        // chunk ahead of their use); issued on every chunk (chunk 0 reloads itself,
        // unused), for the reason given in the forward scan
        {
            const int nn = max(n - 1, 0);
            const size_t un = unit_of(bb, hv, nn, p.Hv, NC);
            rAq.load(ws.Aq + un * C * C);
            rKh.load(ws.Kh + un * C * DK);
            rdo = load_do(nn);
            rA.load(ws.A + un * C * C);
            rQ.load(ws.Qt + un * C * DK);
            rE.load(ws.Et + un * C * DK);
        }
        lds_barrier();
        // dR = A^T dU;  dS = gamma_C . dS + Qt^T dO
        {
            f4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < C / 16; kb += 2)
                acc = x3_step<true, true>(acc, op_tr<SA, true>(AH, AL, 16 * rb, kb), op_row<SU, true>(DUH, DUL, 16 * ob, kb));
            store_acc_t<SU>(acc, DRH, DRL, rb, ob);
#pragma unroll
            for (int s = 0; s < 4; ++s) dRu[(16 * rb + 4 * gg + s) * DV + j0 + 16 * ob + rr] = acc[s];
        }
#pragma unroll
        for (int x = 0; x < NT; ++x) {
            const int id = w * NT + x, cb = id >> 1, jb = id & 1;
#pragma unroll
            for (int s = 0; s < 4; ++s) dS[x][s] *= gcr[x][s];
#pragma unroll
            for (int kb = 0; kb < C / 16; kb += 2)
                dS[x] = x3_step<true, DO_LO>(dS[x], op_tr<SK, true>(K2H, K2L, 16 * cb, kb), op_tr<SO, DO_LO>(OH, OL, 16 * jb, kb));
        }
        lds_barrier();
        // dS -= Et^T dR  (the Et tile holds -Et)
#pragma unroll
        for (int x = 0; x < NT; ++x) {
            const int id = w * NT + x, cb = id >> 1, jb = id & 1;
#pragma unroll
            for (int kb = 0; kb < C / 16; kb += 2)
                dS[x] = x3_step<true, true>(dS[x], op_tr<SK, true>(K1H, K1L, 16 * cb, kb), op_row<SU, true>(DRH, DRL, 16 * jb, kb));
            store_acc_t<SS>(dS[x], DSH, DSL, cb, jb);
        }
        lds_barrier();
        if (n > 0) {
            store_split<C, C, SA>(rAq, AH, AL);
            store_split<C, DK, SK>(rKh, K1H, K1L);
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
// The products over the value columns (dEt, dQt, dKh, dAq, dA) take split
// operands, the value columns in passes of DH (each pass's tiles staged in LDS,
// the sums kept in the accumulators across passes), so that a work-group takes
// 74 KB of LDS and two share a CU; the 64-deep products of dM stay on the float32
// matrix cores.
// ---------------------------------------------------------------------------
template <int DK, int DV> struct ProdLds {
    static constexpr int DH = DV < 64 ? DV : 64;           // value columns per pass
    static constexpr int KP = DH + 8;                      // split row stride (elements)
    static constexpr int S_ = 0, P_ = 2 * DK * KP, O_ = P_ + 2 * C * KP, END = O_ + 2 * C * KP;
    static constexpr int BYTES_SPLIT = END * 2;
    // dM stage, float32 tiles: dA [C][80], A [C][80], A [C][68], X [C][68]
    static constexpr int BYTES_F32 = 4 * (2 * C * 80 + 2 * C * 68);
    static constexpr int BYTES = BYTES_SPLIT > BYTES_F32 ? BYTES_SPLIT : BYTES_F32;
};

template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(256) void g2b_products(Bwd2Args p, Bwd2Workspace ws) {
    typedef ProdLds<DK, DV> PL;
    constexpr int DH = PL::DH, NP = DV / DH, KP = PL::KP, NCB = DK / 16, NS = 3 * NP;
    constexpr int NO = C * DH / 8 / 256;                                  // dO loads per thread and pass
    constexpr bool DO_LO = !std::is_same<TIn, bf16_t>::value;  // dO is exact in bfloat16 for bf16 inputs
    __shared__ __attribute__((aligned(16))) uint16_t lds[PL::BYTES / 2];
    // stage 0: Sn in S, -dR in P, dO in O; stage 1: dS1 in S, U in P, dO in O;
    // stage 2: dU in P, R in O (each for the value columns of one pass); then the
    // float32 tiles of dM from the start
    uint16_t *SH = lds + PL::S_, *SL = SH + DK * KP, *PH = lds + PL::P_, *PLo = PH + C * KP, *OH = lds + PL::O_,
             *OL = OH + C * KP;
    const int u = blockIdx.x, NC = p.NC;
    const int n = u % NC, hv = (u / NC) % p.Hv, bb = u / (NC * p.Hv);
    const int t0 = n * C, L = min(C, p.T - t0);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, rr = lane & 15, gg = lane >> 4;
    const size_t uC = (size_t)u * C, uS = (size_t)u * DK * DV;
    const TIn *dout = static_cast<const TIn *>(p.dout);

    // the next step's tiles, in registers from their global loads to their LDS stores
    RegTile<DK, DH, 256, DV> rS;
    RegTile<C, DH, 256, DV> rP, rO;
    In8<TIn> xo[NO];  // dO (rows past T read the last token and are zeroed at the store)
    RegTile<C, C> rA;
    // step s: stage s / NP over the value columns j0 = DH (s % NP) ..
    auto load_step = [&](int s) {
        const int st = s / NP, j0 = DH * (s % NP);
        if (st < 2) {
            rS.load((st == 0 ? ws.Sn : ws.dS1) + uS + j0);
            rP.load((st == 0 ? ws.dR : ws.U) + uC * DV + j0);
#pragma unroll
            for (int it = 0; it < NO; ++it) {
                const int i = tid + 256 * it, t = i / (DH / 8), j = (i % (DH / 8)) * 8, tl = min(t, L - 1);
                xo[it].load(dout, (((size_t)bb * p.T + t0 + tl) * p.Hv + hv) * DV + j0 + j);
            }
        } else {
            rP.load(ws.dU + uC * DV + j0);
            rO.load(ws.R + uC * DV + j0);
        }
    };
    auto store_step = [&](int s) {
        const int st = s / NP;
        if (st < 2) {
            store_split<DK, DH, KP, DV>(rS, SH, SL);
            store_split<C, DH, KP, DV>(rP, PH, PLo, st == 0 ? -1.f : 1.f);
#pragma unroll
            for (int it = 0; it < NO; ++it) {
                const int i = tid + 256 * it, t = i / (DH / 8), j = (i % (DH / 8)) * 8;
                f4 lo, hi;
                xo[it].get(lo, hi);
                const float on = t < L ? 1.f : 0.f;
                u16x4 h0, l0, h1, l1;
                split4(lo * on, h0, l0);
                split4(hi * on, h1, l1);
                *reinterpret_cast<u16x4 *>(OH + t * KP + j) = h0;
                *reinterpret_cast<u16x4 *>(OH + t * KP + j + 4) = h1;
                if constexpr (DO_LO) {
                    *reinterpret_cast<u16x4 *>(OL + t * KP + j) = l0;
                    *reinterpret_cast<u16x4 *>(OL + t * KP + j + 4) = l1;
                }
            }
        } else {
            store_split<C, DH, KP, DV>(rP, PH, PLo);
            store_split<C, DH, KP, DV>(rO, OH, OL);
        }
    };

    f4 e[NCB], q[NCB], kh[NCB], aq[4], dA[4];
#pragma unroll
    for (int x = 0; x < NCB; ++x) e[x] = q[x] = kh[x] = f4{0, 0, 0, 0};
#pragma unroll
    for (int x = 0; x < 4; ++x) aq[x] = dA[x] = f4{0, 0, 0, 0};
    float dgs = 0.f;  // dgamma_C partial: channel tid / 2, half tid % 2 of each pass's columns

    load_step(0);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int st = s / NP, j0 = DH * (s % NP);
        if (s > 0) lds_barrier();  // the previous step's products are done with the LDS
        store_step(s);
        lds_barrier();
        if (s + 1 < NS) load_step(s + 1);
        if (s + 1 == NS) rA.load(ws.A + uC * C);
        if (st == 0) {
            // dEt = -dR Sn^T, dQt = dO Sn^T; dgamma_C = rowsum(dS1 . Sn)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                mma_x3<DH, KP, KP, true>(e[cb], PH + 16 * w * KP, PLo + 16 * w * KP, SH + 16 * cb * KP,
                                         SL + 16 * cb * KP);
                mma_x3<DH, KP, KP, DO_LO>(q[cb], OH + 16 * w * KP, OL + 16 * w * KP, SH + 16 * cb * KP,
                                          SL + 16 * cb * KP);
            }
            if (tid < 2 * DK) {
                const int c = tid >> 1, h = tid & 1;
                const float *d1 = ws.dS1 + uS + (size_t)c * DV + j0 + h * (DH / 2);
#pragma unroll
                for (int j = 0; j < DH / 2; j += 4) {
                    const f4 x = *reinterpret_cast<const f4 *>(d1 + j);
                    const int o = c * KP + h * (DH / 2) + j;
                    const u16x4 yh = *reinterpret_cast<const u16x4 *>(SH + o), yl = *reinterpret_cast<const u16x4 *>(SL + o);
#pragma unroll
                    for (int k = 0; k < 4; ++k) dgs += x[k] * (bf16_to_f32(yh[k]) + bf16_to_f32(yl[k]));
                }
            }
            if (s % NP == NP - 1) {
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const size_t o = (uC + 16 * w + 4 * gg + x) * DK + 16 * cb + rr;
                        ws.dEt[o] = e[cb][x];
                        ws.dQt[o] = q[cb][x];
                    }
                const float d2 = dgs + __shfl_xor(dgs, 1);
                if (tid < 2 * DK && !(tid & 1)) ws.dgC[(size_t)u * DK + (tid >> 1)] = d2;
            }
        } else if (st == 1) {
            // dKh = U dS1^T, dAq = tril(dO U^T)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                mma_x3<DH, KP, KP, true>(kh[cb], PH + 16 * w * KP, PLo + 16 * w * KP, SH + 16 * cb * KP,
                                         SL + 16 * cb * KP);
#pragma unroll
            for (int ib = 0; ib < 4; ++ib)
                if (ib <= w)
                    mma_x3<DH, KP, KP, DO_LO>(aq[ib], OH + 16 * w * KP, OL + 16 * w * KP, PH + 16 * ib * KP,
                                              PLo + 16 * ib * KP);
            if (s % NP == NP - 1) {
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                    for (int x = 0; x < 4; ++x) ws.dKh[(uC + 16 * w + 4 * gg + x) * DK + 16 * cb + rr] = kh[cb][x];
                float *dAqu = ws.dAq + uC * C;
#pragma unroll
                for (int ib = 0; ib < 4; ++ib)
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const int t = 16 * w + 4 * gg + x, i = 16 * ib + rr;
                        dAqu[t * C + i] = i <= t ? aq[ib][x] : 0.f;
                    }
            }
        } else {
            // dA = dU R^T
#pragma unroll
            for (int ib = 0; ib < 4; ++ib)
                mma_x3<DH, KP, KP, true>(dA[ib], PH + 16 * w * KP, PLo + 16 * w * KP, OH + 16 * ib * KP,
                                         OL + 16 * ib * KP);
        }
    }
    lds_barrier();
    // X = A^T dA; dM = -strict_tril(X A^T), in float32
    float *f32s = reinterpret_cast<float *>(lds);
    float *dAs = f32s, *A80 = f32s + C * 80, *A68 = f32s + 2 * C * 80, *Xs = A68 + C * 68;
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int x = 0; x < 4; ++x) dAs[(16 * w + 4 * gg + x) * 80 + 16 * ib + rr] = dA[ib][x];
    rA.template store<80>(A80);
    rA.template store<68>(A68);
    lds_barrier();
    // X[i][s] = sum_t A[t][i] dA[t][s] (A[t][i] = 0 for t < i): rows i of block w
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
        f4 acc = {0, 0, 0, 0};
        mma<C, 1, 80, 80, 1>(acc, A80 + 16 * w, dAs + 16 * sb);
        dA[sb] = acc;  // reuse the registers for X
    }
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
        for (int x = 0; x < 4; ++x) Xs[(16 * w + 4 * gg + x) * 68 + 16 * sb + rr] = dA[sb][x];
    lds_barrier();
    // dM[i][q] = -sum_s X[i][s] A[q][s] (A[q][s] = 0 for s > q), strictly lower
    float *dMu = ws.dM + uC * C;
    for (int qb = 0; qb < 4; ++qb) {
        f4 acc = {0, 0, 0, 0};
        if (qb <= w) mma<C, 68, 1, 1, 68>(acc, Xs + 16 * w * 68, A68 + 16 * qb * 68);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int i = 16 * w + 4 * gg + x, qq = 16 * qb + rr;
            dMu[i * C + qq] = qq < i ? -acc[x] : 0.f;
        }
    }
}

// ---------------------------------------------------------------------------
// g2b_local: one work-group of 8 waves per (chunk, 32 key channels), the
// channel groups of a chunk on one XCD (their reads of the chunk's dM and dA_qk
// meet in its L2).  Wave w owns 16-token block b = w / 2 and 16-channel tile
// ct = w % 2, in the matrix-core accumulator layout throughout: lane (g, r)
// holds tokens 16 b + 4 g + s (s = 0..3) of channel 16 ct + r.  First the
// block pairs below the diagonal on the matrix cores (rows t of block b
// against every earlier block, rows i of block b against every later block),
// whose accumulators are then the lane's own sums; then the pairs inside block
// b on the vector unit; then the chain rule.  76 KB of LDS and at most 128
// registers: two work-groups share a CU at four waves per SIMD.
// ---------------------------------------------------------------------------
constexpr int LOCAL_NT = 512, LOCAL_CH = 32;

template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(LOCAL_NT, 4) void g2b_local(Bwd2Args p, Bwd2Workspace ws) {
    constexpr int CG = DK / LOCAL_CH, NRG = C / 4;  // channel groups; row groups of 4 tokens
    constexpr int LS = LOCAL_CH + 4;  // channel-tile row stride: a wave's 4 token groups on disjoint banks
    constexpr int MS = C + 4;         // dM / dA_qk row stride
    __shared__ __attribute__((aligned(16))) float Gs[C * LS], Ks[C * LS], Es[C * LS], Qs[C * LS], dMs[C * MS],
        dAqs[C * MS], blk[NRG * LOCAL_CH], gcp[NRG * LOCAL_CH], alp[NRG * LOCAL_CH];
    // work-group -> (unit, channel group): work-group i runs on XCD i % 8, so units go
    // eight at a time across the XCDs with the channel groups of each on one of them
    const int units = p.B * p.Hv * p.NC, full = units / 8 * 8 * CG;
    int u, cg;
    if ((int)blockIdx.x < full) {
        const int j = blockIdx.x / 8;
        u = 8 * (j / CG) + (int)blockIdx.x % 8;
        cg = j % CG;
    } else {
        const int r = (int)blockIdx.x - full;
        u = units / 8 * 8 + r / CG;
        cg = r % CG;
    }
    const int NC = p.NC;
    const int n = u % NC, hv = (u / NC) % p.Hv, bb = u / (NC * p.Hv), hk = hv / (p.Hv / p.Hk);
    const int t0 = n * C, L = min(C, p.T - t0);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, rr = lane & 15, gg = lane >> 4;
    const int b = w >> 1, ct = w & 1, cc = 16 * ct + rr, c = LOCAL_CH * cg + cc;
    const int r0 = 16 * b + 4 * gg, rgi = 4 * b + gg;  // the lane's first token; its row group
    const TIn *q = static_cast<const TIn *>(p.q), *k = static_cast<const TIn *>(p.k);
    const TIn *a = static_cast<const TIn *>(p.a), *er = static_cast<const TIn *>(p.erase);
    const float Al = p.A_log[(size_t)hv * DK + c], rate = exp_fast(Al);

    // dM and dA_qk tiles, loaded with the rest and stored to LDS after the gates
    RegTile<C, C, LOCAL_NT> rM, rAq;
    rM.load(ws.dM + (size_t)u * C * C);
    rAq.load(ws.dAq + (size_t)u * C * C);

    // gates of the lane's tokens; the in-chunk prefix of g runs over them, then the
    // totals of the earlier row groups are added (the logits a and the erase gate
    // stay in registers for the chain rule)
    float grun = 0.f, gpre[4], a_row[4], beta_row[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const int t = r0 + x, tl = min(t, L - 1);
        const size_t kq = (((size_t)bb * p.T + t0 + tl) * p.Hk + hk) * DK + c;
        const size_t ka = (((size_t)bb * p.T + t0 + tl) * p.Hv + hv) * DK + c;
        const float on = t < L ? 1.f : 0.f;
        const float kv = io<TIn>::ld(k, kq) * on;
        a_row[x] = io<TIn>::ld(a, ka);
        beta_row[x] = sigmoid_fast(io<TIn>::ld(er, ka));
        grun += -rate * softplus_fast(a_row[x]) * LOG2E * on;
        gpre[x] = grun;
        Ks[t * LS + cc] = kv;
        Es[t * LS + cc] = beta_row[x] * kv;
        Qs[t * LS + cc] = p.scale * io<TIn>::ld(q, kq) * on;
    }
    blk[rgi * LOCAL_CH + cc] = grun;
    rM.template store<MS>(dMs);
    rAq.template store<MS>(dAqs);
    __syncthreads();
    {
        float off = 0.f;
        for (int x = 0; x < rgi; ++x) off += blk[x * LOCAL_CH + cc];
#pragma unroll
        for (int x = 0; x < 4; ++x) Gs[(r0 + x) * LS + cc] = gpre[x] + off;
    }
    __syncthreads();

    // inputs of the chain rule, in flight during the pair sums
    const size_t ub = (size_t)u * C * DK;
    float pdE[4], pdQ[4], pdK[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        pdE[x] = ws.dEt[ub + (r0 + x) * DK + c];
        pdQ[x] = ws.dQt[ub + (r0 + x) * DK + c];
        pdK[x] = ws.dKh[ub + (r0 + x) * DK + c];
    }
    const float pgC = ws.dgC[(size_t)u * DK + c];

    // block pairs below the diagonal (MFMA: lane supplies A[rr][gg], B[gg][rr]; the
    // accumulator element s is token 16 b + 4 gg + s, channel cc):
    //   rows t of block b, reference r = 16 b (i < r <= t):
    //     de_t  = e^{G_t - G_r} sum_{i < r} dM_ti  k_i e^{G_r - G_i}, dqs_t likewise with dAq
    //   rows i of block b, each later block b2 with reference r = 16 b2:
    //     dk_i += e^{G_r - G_i} sum_{t in b2} dM_ti e_t e^{G_t - G_r} + dAq_ti qs_t e^{G_t - G_r}
    f4 sde = {0, 0, 0, 0}, sdq = {0, 0, 0, 0}, sdk = {0, 0, 0, 0};
    if (b > 0) {
        const int r = 16 * b;
        const float Gr = Gs[r * LS + cc];
        // kept rolled: unrolled by whole 16-row blocks it measured slower
#pragma unroll 1
        for (int i0 = 0; i0 < r; i0 += 4) {
            const int i = i0 + gg;
            const float bv = Ks[i * LS + cc] * ex2(Gr - Gs[i * LS + cc]);
            sde = mfma_f32_k4(dMs[(r + rr) * MS + i], bv, sde);
            sdq = mfma_f32_k4(dAqs[(r + rr) * MS + i], bv, sdq);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float F = ex2(Gs[(r0 + s) * LS + cc] - Gr);
            sde[s] *= F;
            sdq[s] *= F;
        }
    }
    for (int b2 = b + 1; b2 < 4; ++b2) {
        const int r = 16 * b2;
        const float Gr = Gs[r * LS + cc];
        f4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) {
            const int t = r + k0 + gg;
            const float f = ex2(Gs[t * LS + cc] - Gr);
            acc = mfma_f32_k4(dMs[t * MS + 16 * b + rr], Es[t * LS + cc] * f, acc);
            acc = mfma_f32_k4(dAqs[t * MS + 16 * b + rr], Qs[t * LS + cc] * f, acc);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) sdk[s] += acc[s] * ex2(Gr - Gs[(r0 + s) * LS + cc]);
    }

    // pairs inside block b, for each of the lane's tokens t and every token o of the
    // block: as t (o <= t) the de, dqs sums, as i (o >= t) the dk sum.  Both sides are
    // summed for every pair: dM (strictly lower) and dA_qk (lower) are zero where a side
    // does not apply, and e^{-|G_t - G_o|} is the decay factor of either side (G does
    // not increase along the chunk).  dM[o][t..t+3], dA_qk[o][t..t+3]: one read each.
    {
        float Gt[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) Gt[s] = Gs[(r0 + s) * LS + cc];
#pragma unroll
        for (int j0 = 0; j0 < 16; j0 += 4) {
            const int o0 = 16 * b + j0;
            f4 mt[4], qt[4];  // dM[t][o0..o0+3], dA_qk[t][o0..o0+3] for the lane's tokens t
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                mt[s] = *reinterpret_cast<const f4 *>(dMs + (r0 + s) * MS + o0);
                qt[s] = *reinterpret_cast<const f4 *>(dAqs + (r0 + s) * MS + o0);
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int o = o0 + jj;
                const float Go = Gs[o * LS + cc], ko = Ks[o * LS + cc], qo = Qs[o * LS + cc], eo = Es[o * LS + cc];
                const f4 mo = *reinterpret_cast<const f4 *>(dMs + o * MS + r0);   // dM[o][t]
                const f4 qq = *reinterpret_cast<const f4 *>(dAqs + o * MS + r0);  // dA_qk[o][t]
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const float E = ex2(-fabsf(Gt[s] - Go)), kE = ko * E;
                    sde[s] += mt[s][jj] * kE;
                    sdq[s] += qt[s][jj] * kE;
                    sdk[s] += (qq[s] * qo + mo[s] * eo) * E;
                }
            }
        }
    }

    // chain rule for the lane's tokens
    const float GC = Gs[(C - 1) * LS + cc];
    float dG[4], de[4], dq[4], dk[4], sKK = 0.f, bsum = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const int t = r0 + x;
        const float G = Gs[t * LS + cc], eg = ex2(G), kg = ex2(GC - G);
        const float dEt = pdE[x], dQt = pdQ[x], dKh = pdK[x];
        const float e = Es[t * LS + cc], qs = Qs[t * LS + cc], kk = Ks[t * LS + cc];
        const float te = sde[x], tq = sdq[x], ik = sdk[x];
        de[x] = eg * dEt + te;
        dq[x] = eg * dQt + tq;
        dk[x] = kg * dKh + ik;
        const float khv = kk * kg;
        dG[x] = dEt * (e * eg) + dQt * (qs * eg) - dKh * khv + e * te + qs * tq - kk * ik;
        sKK += dKh * khv;
        bsum += dG[x];
    }
    blk[rgi * LOCAL_CH + cc] = bsum;
    gcp[rgi * LOCAL_CH + cc] = sKK;
    __syncthreads();
    // dg_t = sum_{r >= t} dG_r; G_C (the last row) also enters through K-hat and gamma_C
    float carry = pgC * ex2(GC);
#pragma unroll
    for (int x = 0; x < NRG; ++x) carry += gcp[x * LOCAL_CH + cc];
    for (int x = rgi + 1; x < NRG; ++x) carry += blk[x * LOCAL_CH + cc];
    float alsum = 0.f;
#pragma unroll
    for (int x = 3; x >= 0; --x) {
        carry += dG[x];
        const int t = r0 + x;
        if (t < L) {
            const size_t ka = (((size_t)bb * p.T + t0 + t) * p.Hv + hv) * DK + c;
            const float av = a_row[x], beta = beta_row[x];
            const float kk = Ks[t * LS + cc];
            const float dg = carry;  // natural-log units
            p.da[ka] = -dg * rate * sigmoid_fast(av);
            alsum += dg * (-rate * softplus_fast(av));
            p.derase[ka] = de[x] * kk * beta * (1.f - beta);
            ws.dqh[ka] = p.scale * dq[x];
            ws.dkh[ka] = dk[x] + de[x] * beta;
        }
    }
    alp[rgi * LOCAL_CH + cc] = alsum;
    __syncthreads();
    if (tid < LOCAL_CH) {
        float sa = 0.f;
#pragma unroll
        for (int x = 0; x < NRG; ++x) sa += alp[x * LOCAL_CH + tid];
        ws.dAl[(size_t)u * DK + LOCAL_CH * cg + tid] = sa;
    }
    // dz = dR -> dv, d_write for the group's share of the value columns
    {
        constexpr int DVG = DV / CG, ITEMS = C * DVG / 8, NIT = (ITEMS + LOCAL_NT - 1) / LOCAL_NT;
        static_assert(DVG % 8 == 0, "value columns per channel group");
        const TIn *v = static_cast<const TIn *>(p.v), *wr = static_cast<const TIn *>(p.write);
        const float *dRu = ws.dR + (size_t)u * C * DV;
        // every load of the loop first (the stores to dv and d_write could alias them)
        In8<TIn> xv[NIT], xw[NIT];
        f4 dzl[NIT][2];
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int i = tid + LOCAL_NT * it, t = i / (DVG / 8), j = DVG * cg + (i % (DVG / 8)) * 8,
                      tl = min(t, L - 1);
            if (i < ITEMS) {
                const size_t kv = (((size_t)bb * p.T + t0 + tl) * p.Hv + hv) * DV + j;
                xv[it].load(v, kv);
                xw[it].load(wr, kv);
                dzl[it][0] = *reinterpret_cast<const f4 *>(dRu + t * DV + j);
                dzl[it][1] = *reinterpret_cast<const f4 *>(dRu + t * DV + j + 4);
            }
        }
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int i = tid + LOCAL_NT * it, t = i / (DVG / 8), j = DVG * cg + (i % (DVG / 8)) * 8,
                      tl = min(t, L - 1);
            if (i < ITEMS && t < L) {
                const size_t kv = (((size_t)bb * p.T + t0 + tl) * p.Hv + hv) * DV + j;
                f4 vv[2], om[2];
                xv[it].get(vv[0], vv[1]);
                xw[it].get(om[0], om[1]);
                const f4 (&dz)[2] = dzl[it];
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

// T = 0: dS0 = dS_T (or 0), dA_log = 0; B = 0 (ns = 0): dA_log = 0
__global__ void g2b_empty(float *dS0, const float *dST, size_t ns, float *dA_log, size_t na) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < ns + na; i += (size_t)gridDim.x * blockDim.x) {
        if (i < ns) {
            if (dS0) dS0[i] = dST ? dST[i] : 0.f;
        } else {
            dA_log[i - ns] = 0.f;
        }
    }
}

template <typename TIn, int DK, int DV>
hipError_t launch_bwd2_t(const Bwd2Args &p, const Bwd2Workspace &ws, hipStream_t s, const hipEvent_t *ev) {
    const unsigned units = (unsigned)(p.B * p.Hv * p.NC), slices = (unsigned)(p.B * p.Hv * (DV / 32));
    hipError_t e = hipSuccess;
    auto rec = [&](int i) {
        if (ev && e == hipSuccess) e = hipEventRecord(ev[i], s);
    };
    rec(0);
    hipLaunchKernelGGL((g2b_prep<TIn, DK, DV>), dim3(units), dim3(PREP_NT), 0, s, p, ws);
    rec(1);
    hipLaunchKernelGGL((g2b_fwd_scan<TIn, DK, DV>), dim3(slices), dim3(SCAN_NT), 0, s, p, ws);
    rec(2);
    hipLaunchKernelGGL((g2b_bwd_scan<TIn, DK, DV>), dim3(slices), dim3(SCAN_NT), 0, s, p, ws);
    rec(3);
    hipLaunchKernelGGL((g2b_products<TIn, DK, DV>), dim3(units), dim3(256), 0, s, p, ws);
    rec(4);
    hipLaunchKernelGGL((g2b_local<TIn, DK, DV>), dim3(units * (DK / LOCAL_CH)), dim3(LOCAL_NT), 0, s, p, ws);
    rec(5);
    const size_t nq = (size_t)p.B * p.T * p.Hk * DK / 256 + 1;
    hipLaunchKernelGGL((g2b_reduce<DK>), dim3((unsigned)(nq < 65536 ? nq : 65536)), dim3(256), 0, s, p, ws);
    rec(6);
    const hipError_t le = hipGetLastError();
    return le != hipSuccess ? le : e;
}

}  // namespace

// Buffers whose lives do not overlap share memory.  Lives (W = written, R = read):
//   A: prep W, fwd/bwd scans and products R (products last);  Aq, Et, Qt, Kh, gC: prep W, scans R;
//   Sn, R, U: forward scan W, products R;
//   dS1, dU: reverse scan W, products R;  dR: reverse scan W, products and local R;
//   dEt, dQt, dKh, dgC, dAq, dM: products W, local R;  dqh, dkh, dAl: local W, reduce R.
// So products writes into the space of buffers last read by the scans (dEt into Et, dQt
// into Qt, dKh into Kh, dgC into gC, dAq into Aq) or by itself (dM into A: a work-group
// reads its chunk's A before it writes that chunk's dM), and local into the
// space of buffers last read by products (dqh into Sn, dkh into dS1, dAl into U).  The
// only kernel that writes the space of a buffer it reads is products (dM over A), each
// work-group in its own chunk's part, after its last read of it.
size_t bwd2_workspace_layout(int B, int T, int Hv, int Dk, int Dv, void *base, Bwd2Workspace *ws) {
    const size_t NC = ((size_t)T + C - 1) / C, U = (size_t)B * Hv * NC;
    size_t off = 0;
    auto take = [&](size_t elems) {
        float *p = base ? reinterpret_cast<float *>(static_cast<char *>(base) + off) : nullptr;
        off += (elems * 4 + 255) / 256 * 256;
        return p;
    };
    Bwd2Workspace w{};
    w.A = w.dM = take(U * C * C);
    w.Aq = w.dAq = take(U * C * C);
    w.Et = w.dEt = take(U * C * Dk);
    w.Qt = w.dQt = take(U * C * Dk);
    w.Kh = w.dKh = take(U * C * Dk);
    w.gC = w.dgC = take(U * Dk);
    w.R = take(U * C * Dv);
    w.U = w.dAl = take(U * C * Dv);   // dAl: Dk per unit
    w.dU = take(U * C * Dv);
    w.dR = take(U * C * Dv);
    // dqh / dkh hold [B][T][Hv][Dk]: at most U * C * Dk floats, within S_n / dS_{n+1} (Dv >= 64 = C)
    w.Sn = w.dqh = take(U * Dk * Dv);
    w.dS1 = w.dkh = take(U * Dk * Dv);
    w.bytes = off;
    if (ws) *ws = w;
    return off;
}

hipError_t launch_bwd2(const Bwd2Args &p, const Bwd2Workspace &ws, hipStream_t s, const hipEvent_t *ev) {
    if (p.B == 0 || p.T == 0) {  // no tokens: dA_log (a sum over none) is zero
        const size_t ns = (size_t)p.B * p.Hv * p.Dk * p.Dv, na = (size_t)p.Hv * p.Dk;
        hipLaunchKernelGGL(g2b_empty, dim3((unsigned)((ns + na) / 256 + 1 < 65536 ? (ns + na) / 256 + 1 : 65536)),
                           dim3(256), 0, s, p.dS0, p.dST, ns, p.dA_log, na);
        return hipGetLastError();
    }
    if (p.f32) {
        if (p.Dk == 128 && p.Dv == 128) return launch_bwd2_t<float, 128, 128>(p, ws, s, ev);
        if (p.Dk == 128 && p.Dv == 64) return launch_bwd2_t<float, 128, 64>(p, ws, s, ev);
        if (p.Dk == 64 && p.Dv == 128) return launch_bwd2_t<float, 64, 128>(p, ws, s, ev);
        if (p.Dk == 64 && p.Dv == 64) return launch_bwd2_t<float, 64, 64>(p, ws, s, ev);
        return hipErrorInvalidValue;
    }
    if (p.Dk == 128 && p.Dv == 128) return launch_bwd2_t<bf16_t, 128, 128>(p, ws, s, ev);
    if (p.Dk == 128 && p.Dv == 64) return launch_bwd2_t<bf16_t, 128, 64>(p, ws, s, ev);
    if (p.Dk == 64 && p.Dv == 128) return launch_bwd2_t<bf16_t, 64, 128>(p, ws, s, ev);
    if (p.Dk == 64 && p.Dv == 64) return launch_bwd2_t<bf16_t, 64, 64>(p, ws, s, ev);
    return hipErrorInvalidValue;
}

}  // namespace gdn
