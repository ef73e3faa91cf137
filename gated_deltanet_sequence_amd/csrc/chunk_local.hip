// chunk_local.hip -- gate preparation and the chunk-local WY auxiliaries of the
// chunked prefill (method and notation in prefill_common.h).  Fully parallel
// over chunks: one work-group of 4 waves per (sequence, key head, chunk).
//
//  1. Q and K rows of the chunk are converted to the operand type and staged in
//     LDS as swizzled tile images; the images of Q and K (and K^T for float32
//     operands) are written to the workspace for the scan, which copies them
//     into LDS byte for byte.
//     The read-out scale is folded into Q here, so Q S and A_qk (every term of
//     the output) carry it and the scan applies none.
//  2. K K^T and Q K^T (lower-triangular 16x16 tiles) on the matrix cores, once
//     per key head: they are shared by its Hv/Hk value heads.
//  3. Per value head (one wave each): gate preparation -- g = -exp(A_log)
//     softplus(a + dt_bias) and beta = sigmoid(b) in float32 (dingfen.github.io
//     page, sections 9-10) and the in-chunk inclusive prefix sum G of g in
//     float64, so that e^{G_r - G_i} keeps float32 accuracy when |G| is in the
//     hundreds; the decay ratios Gamma = e^{G_r - G_i} of the lower triangle
//     (computed once, shared by L and A_qk); L = beta Gamma (.) K K^T; the
//     blocked inverse A = (I + L)^{-1} (diagonal 16x16 blocks by forward
//     substitution in registers, off-diagonal blocks on the matrix cores); and
//     the operand fragments of the two matrices the scan applies to its
//     residual (A and A_qk with the per-token factors folded in) plus the
//     per-token decay record.
#include <utility>

#include "prefill_common.h"

namespace gdn {

size_t prefill_workspace_layout(int B, int T, int Hk, int Hv, int Dk, bool f32, void *base,
                                PrefillWorkspace *ws) {
    const size_t NC = (size_t)(T + C - 1) / C;
    const size_t vunits = (size_t)B * Hv * NC, kunits = (size_t)B * Hk * NC;
    const size_t esz = f32 ? 4 : 2;
    size_t off = 0;
    const size_t oT = off;  off = align256(off + vunits * C * 2 * sizeof(float));
    const size_t oA = off;  off = align256(off + vunits * NPAIR * 64 * 8 * esz);
    const size_t oQ = off;  off = align256(off + vunits * NPAIR * 64 * 8 * esz);
    const size_t oQi = off; off = align256(off + kunits * C * Dk * esz);
    const size_t oKi = off; off = align256(off + kunits * C * Dk * esz);
    // K^T images only for float32 operands: the float16 scan reads K^T operands
    // from the K image with transposed LDS reads
    const size_t oTi = off; off = align256(off + (f32 ? kunits * C * Dk * esz : 0));
    if (ws) {
        char *p = (char *)base;
        ws->tok = (float *)(p + oT);
        ws->apair = p + oA;
        ws->qpair = p + oQ;
        ws->qimg = p + oQi;
        ws->kimg = p + oKi;
        ws->timg = f32 ? p + oTi : nullptr;
        ws->bytes = off;
    }
    return off;
}

// Logical column of physical position p (inverse of perm_col).
template <bool F32>
__device__ __forceinline__ int unperm_col(int p) {
    if constexpr (F32) return p;
    return (p & ~31) | (((p & 7) >> 2) << 4) | (((p & 31) >> 3) << 2) | (p & 3);
}

template <bool F32, int DK>
struct ChunkLocalCfg {
    typedef typename mma<F32>::E E;
    static constexpr size_t IMG = (size_t)C * DK;                  // elements per image
    // per-wave scratch: the 10 lower 16x16 blocks of X = (I + L)^{-1}, then G
    // (64 doubles) and beta; the diagonal blocks of L live in the off-diagonal
    // X slots until the off-diagonal blocks of X are formed (LDS stays under
    // 80 KB: two work-groups per CU)
    static constexpr size_t WAVE_FLOATS = 10 * 256 + 128 + 64;
    static constexpr size_t IMG_BYTES = 2 * IMG * sizeof(E);
    static constexpr size_t WAVE_BYTES = 4 * WAVE_FLOATS * sizeof(float);
    static constexpr size_t U_BYTES = IMG_BYTES > WAVE_BYTES ? IMG_BYTES : WAVE_BYTES;
};

template <bool F32, typename TIn, int DK>
__global__ __launch_bounds__(256, F32 ? 1 : 2) void chunk_local_kernel(
    int B, int T, int Hk, int Hv, int NC, float scale, const TIn *__restrict__ q, const TIn *__restrict__ k,
    const float *__restrict__ a, const float *__restrict__ b, const float *__restrict__ A_log,
    const float *__restrict__ dt_bias, float *__restrict__ tok, typename mma<F32>::E *__restrict__ apair,
    typename mma<F32>::E *__restrict__ qpair, typename mma<F32>::E *__restrict__ qimg,
    typename mma<F32>::E *__restrict__ kimg, typename mma<F32>::E *__restrict__ timg) {
    typedef ChunkLocalCfg<F32, DK> CF;
    typedef typename mma<F32>::E E;
    typedef typename mma<F32>::V4 V4;
    constexpr int EPG = img_epg<F32>();
    constexpr size_t IMG = CF::IMG;

    // union: Q/K images (steps 1-2) | per-wave scratch (step 3)
    __shared__ __attribute__((aligned(16))) char u_raw[CF::U_BYTES];
    __shared__ __attribute__((aligned(16))) float KKt[10 * 256];
    __shared__ __attribute__((aligned(16))) float QKt[10 * 256];
    E *Qi = reinterpret_cast<E *>(u_raw);
    E *Ki = Qi + IMG;

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in a scalar register
    const int G = Hv / Hk;
    const int units = B * Hk * NC;

    // Persistent: the work-group walks units u = (b, key head, chunk), and the
    // next unit's global loads (Q and K rows, gate logits and parameters of
    // this wave's first value head) are in flight while this unit computes.
    // The rows stay raw 16-byte pieces until the next unit's images are
    // written, and they are loaded without a branch: a row past the sequence
    // end loads the tensor's first piece and is zeroed at conversion (rmask).
    // Converting inside a bounds branch made the compiler wait for every
    // piece right where it was loaded, one memory round trip after another.
    constexpr int NPC = C * (DK / 8) / 256;  // 8-element pieces of Q (and of K) per thread
    constexpr int LPP = (int)sizeof(TIn) / 2;  // 16-byte loads per 8-element piece
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    u4v qr[NPC][LPP], kr[NPC][LPP];
    unsigned rmask = 0;  // bit it: piece it lies in a row before the sequence end
    float a_pre = 0.f, b_pre = 0.f, alog_pre = 0.f, dtb_pre = 0.f;
    auto prefetch = [&](int u) {
        const int n = u % NC, hk = (u / NC) % Hk, bb = u / (NC * Hk);
        const int t0 = n * C;
        rmask = 0;
#pragma unroll
        for (int it = 0; it < NPC; ++it) {
            const int idx = tid + 256 * it, r = idx / (DK / 8), c8 = (idx % (DK / 8)) * 8;
            const bool ok = t0 + r < T;
            rmask |= ok ? 1u << it : 0u;
            const size_t off = ok ? (((size_t)bb * T + t0 + r) * Hk + hk) * DK + c8 : 0;
#pragma unroll
            for (int l = 0; l < LPP; ++l) {
                qr[it][l] = *reinterpret_cast<const u4v *>(q + off + 4 * l);
                kr[it][l] = *reinterpret_cast<const u4v *>(k + off + 4 * l);
            }
        }
        a_pre = b_pre = 0.f;
        if (w < G) {
            const int hv = hk * G + w;
            alog_pre = A_log[hv];
            dtb_pre = dt_bias[hv];
            if (t0 + lane < T) {
                const size_t ia = ((size_t)bb * T + t0 + lane) * Hv + hv;
                a_pre = a[ia];
                b_pre = b[ia];
            }
        }
    };
    // raw piece -> 8 values (zero when the row lies past the sequence end)
    auto unpack = [&](const u4v (&r)[LPP], bool ok, f4 &lo, f4 &hi) {
        if constexpr (LPP == 2) {
            lo = ok ? __builtin_bit_cast(f4, r[0]) : f4{0, 0, 0, 0};
            hi = ok ? __builtin_bit_cast(f4, r[1]) : f4{0, 0, 0, 0};
        } else {
            const u4v z = ok ? r[0] : u4v{0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                lo[2 * j] = __uint_as_float(z[j] << 16);
                lo[2 * j + 1] = __uint_as_float(z[j] & 0xffff0000u);
                hi[2 * j] = __uint_as_float(z[2 + j] << 16);
                hi[2 * j + 1] = __uint_as_float(z[2 + j] & 0xffff0000u);
            }
        }
    };

    if ((int)blockIdx.x >= units) return;
    prefetch(blockIdx.x);
    for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int n = u % NC, hk = (u / NC) % Hk, bb = u / (NC * Hk);
    const int t0 = n * C;
    const size_t ku = (size_t)u;

    // ---- 1. Q and K of this unit (zero past the end) into LDS as images
#pragma unroll
    for (int it = 0; it < NPC; ++it) {
        const int idx = tid + 256 * it, r = idx / (DK / 8), c8 = (idx % (DK / 8)) * 8;
        const bool ok = (rmask >> it) & 1u;
        f4 ql, qh, kl, kh;
        unpack(qr[it], ok, ql, qh);
        unpack(kr[it], ok, kl, kh);
        *reinterpret_cast<V4 *>(Qi + img_index<F32>(r, DK, perm_col<F32>(c8))) = mma<F32>::from_f4(scale * ql);
        *reinterpret_cast<V4 *>(Qi + img_index<F32>(r, DK, perm_col<F32>(c8 + 4))) = mma<F32>::from_f4(scale * qh);
        *reinterpret_cast<V4 *>(Ki + img_index<F32>(r, DK, perm_col<F32>(c8))) = mma<F32>::from_f4(kl);
        *reinterpret_cast<V4 *>(Ki + img_index<F32>(r, DK, perm_col<F32>(c8 + 4))) = mma<F32>::from_f4(kh);
    }
    const float a_cur = a_pre, b_cur = b_pre, alog_cur = alog_pre, dtb_cur = dtb_pre;
    if (u + (int)gridDim.x < units) prefetch(u + gridDim.x);
    __syncthreads();

    // ---- images to the workspace: Q and K verbatim, K^T transposed (float32)
    {
        typedef uint32_t u4v __attribute__((ext_vector_type(4)));
        const u4v *src = reinterpret_cast<const u4v *>(u_raw);
        u4v *dq = reinterpret_cast<u4v *>(qimg + ku * IMG);
        u4v *dk = reinterpret_cast<u4v *>(kimg + ku * IMG);
        constexpr int UNITS = (int)(IMG * sizeof(E) / 16);
        static_assert(UNITS % 256 == 0, "whole 16-byte pieces per thread");
#pragma unroll
        for (int it = 0; it < UNITS / 256; ++it) {  // a fixed count: the compiler counts these stores
            const int i = tid + 256 * it;
            dq[i] = src[i];
            dk[i] = src[UNITS + i];
        }
        if constexpr (F32) {
            E *dt = timg + ku * IMG;
            constexpr int GPR = C / EPG;  // 16-byte groups per K^T row
            for (int job = tid; job < DK * GPR; job += 256) {
                const int R = job / GPR, gp = job % GPR;
                const int pr = perm_col<F32>(R);
                E vals[EPG];
#pragma unroll
                for (int j = 0; j < EPG; ++j) {
                    const int tk = unperm_col<F32>(gp * EPG + j);
                    vals[j] = Ki[img_index<F32>(tk, DK, pr)];
                }
                *reinterpret_cast<u4v *>(dt + img_index<F32>(R, C, gp * EPG)) = *reinterpret_cast<const u4v *>(vals);
            }
        }
    }

    // ---- 2. K K^T and Q K^T, lower-triangular 16x16 tiles (10 each): wave w
    //      takes the row tiles {3, 0} (w < 2) or {2, 1} (5 tiles either way) of
    //      K K^T (even w) or Q K^T (odd w), reading each row tile's operands
    //      once.  Tile (rt, ct) of X K^T is formed as K_ct X_rt^T, whose
    //      accumulator holds row 16rt + m, columns 16ct + 4g .. +3 -- the
    //      operand layout its readers load, stored with one 16-byte write.
    {
        const E *X = (w & 1) ? Qi : Ki;
        float *Dst = (w & 1) ? QKt : KKt;
        for (int h = 0; h < 2; ++h) {
            const int rt = w < 2 ? (h == 0 ? 3 : 0) : (h == 0 ? 2 : 1);
            V4 xa[DK / 32][2];
#pragma unroll
            for (int kq = 0; kq < DK / 32; ++kq) img_pair<F32>(X, DK, 16 * rt + m, kq, g, xa[kq][0], xa[kq][1]);
            for (int ct = 0; ct <= rt; ++ct) {
                f4 acc = {0, 0, 0, 0};
#pragma unroll
                for (int kq = 0; kq < DK / 32; ++kq) {
                    V4 b0, b1;
                    img_pair<F32>(Ki, DK, 16 * ct + m, kq, g, b0, b1);
                    acc = mma<F32>::pair(acc, b0, b1, xa[kq][0], xa[kq][1]);
                }
                *reinterpret_cast<f4 *>(Dst + tri_index(rt, ct) * 256 + m * 16 + 4 * g) = acc;
            }
        }
    }
    __syncthreads();  // the images in LDS are dead from here on

    // ---- 3. per value head, one wave each
    float *Xw = reinterpret_cast<float *>(u_raw) + w * CF::WAVE_FLOATS;
    double *Gs = reinterpret_cast<double *>(Xw + 10 * 256);
    // diagonal block rb of L, in off-diagonal X slot (1,0), (2,0), (2,1) or (3,0)
    auto Ld = [&](int rb) { return Xw + (rb == 0 ? 1 : rb == 1 ? 3 : rb == 2 ? 4 : 6) * 256; };
    float *Bs = reinterpret_cast<float *>(Gs + 64);
    for (int j = w; j < G; j += 4) {
        const int hv = hk * G + j;
        const size_t vu = ((size_t)bb * Hv + hv) * NC + n;

        // gates: lane = token
        const int t = t0 + lane;
        float gl = 0.f, be = 0.f;
        if (t < T) {
            float av = a_cur, bv = b_cur, alog = alog_cur, dtb = dtb_cur;
            if (j != w) {
                const size_t ia = ((size_t)bb * T + t) * Hv + hv;
                av = a[ia];
                bv = b[ia];
                alog = A_log[hv];
                dtb = dt_bias[hv];
            }
            if constexpr (F32) {
                gl = -expf(alog) * softplus_f32(av + dtb);
                be = sigmoid_f32(bv);
            } else {
                gl = -exp_fast(alog) * softplus_fast(av + dtb);
                be = sigmoid_fast(bv);
            }
        }
        const double Gd = wave_prefix_sum_f64((double)gl);
        const double Glast = __longlong_as_double(
            ((long long)__builtin_amdgcn_readlane((int)(__double_as_longlong(Gd) >> 32), 63) << 32) |
            (unsigned)__builtin_amdgcn_readlane((int)__double_as_longlong(Gd), 63));
        Gs[lane] = Gd;
        Bs[lane] = be;
        {   // token record: gamma = e^G in token order, then again with token
            // 16r + m at position 4m + r
            float *tr = tok + vu * C * 2;
            const float gam = __expf((float)Gd);
            tr[lane] = gam;
            tr[64 + 4 * (lane & 15) + (lane >> 4)] = gam;
        }
        wave_lds_sync();

        // decay ratios of the strictly-lower triangle in A-operand layout:
        // lane (m, g) of block (rb, kb) holds rows 16rb+m, columns 16kb+4g+s
        f4 Gm[10];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const int row = 16 * rb + m;
            const double Gr = Gs[row];
#pragma unroll
            for (int kb = 0; kb <= rb; ++kb)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int col = 16 * kb + 4 * g + s;
                    Gm[tri_index(rb, kb)][s] = col < row ? __expf((float)(Gr - Gs[col])) : 0.f;
                }
        }
        // L: off-diagonal blocks as operand fragments, diagonal blocks row-major in Ld
        f4 Lf[10];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const float br = Bs[16 * rb + m];
#pragma unroll
            for (int kb = 0; kb <= rb; ++kb) {
                const int ti = tri_index(rb, kb);
                const f4 kk = *reinterpret_cast<const f4 *>(KKt + ti * 256 + m * 16 + 4 * g);
                const f4 lv = br * Gm[ti] * kk;
                if (kb < rb) Lf[ti] = lv;
                else *reinterpret_cast<f4 *>(Ld(rb) + m * 16 + 4 * g) = lv;
            }
        }
        wave_lds_sync();

        // diagonal blocks of X: lane (block bq, column c) by forward substitution,
        // column-oriented: with x = column c of X (x[r] = delta_rc to start),
        // for j = 0..14, x[r] -= L[r][j] x[j] for r > j.  Each lane keeps column
        // c of L in registers; L[r][j] comes from lane j of the same 16-lane
        // row (the block) by a DPP row broadcast inside the multiply-add, so
        // the inner step is one vector instruction with no LDS access.
        {
            const int bq = lane >> 4, c = lane & 15;
            const float *Lb = Ld(bq);
            float lv[16], x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                lv[r] = Lb[r * 16 + c];
                x[r] = (r == c) ? 1.f : 0.f;
            }
            subst_steps(lv, x, std::make_integer_sequence<int, 15>());
#pragma unroll
            for (int r = 0; r < 16; ++r) Xw[tri_index(bq, bq) * 256 + r * 16 + c] = x[r];
        }
        wave_lds_sync();

        f4 xt[10];  // A^T blocks (kb, mb) as A operands: lane holds A[16mb+4g+s][16kb+m]
        inverse_offdiag<F32>(Xw, Lf, m, g, xt);
        wave_lds_sync();

        // Operand fragments of the two per-chunk matrices the scan applies to the
        // residual R' = V - gamma (.) (K S):
        //   Ae = diag(eta) A diag(beta)         -> eta (.) Delta = Ae R'
        //   Ao = A_qk A diag(beta)              -> A_qk Delta    = Ao R'
        // with A = (I + L)^{-1} (unit diagonal; Xw) and A_qk = Gamma (.) Q K^T
        // including its diagonal.  Both are lower triangular with diagonal.
        // Ao's blocks come from the matrix cores as Ao^T = A^T A_qk^T, whose
        // accumulator tile is exactly the A-operand layout of Ao.
        f4 aq[10];  // A_qk blocks (rb, kb), A-operand layout (row 16rb+m, columns 16kb+4g+s)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int kb = 0; kb <= rb; ++kb) {
                const int ti = tri_index(rb, kb);
                f4 gm = Gm[ti];
                if (kb == rb)
#pragma unroll
                    for (int s = 0; s < 4; ++s) gm[s] = (4 * g + s == m) ? 1.f : gm[s];
                aq[ti] = gm * *reinterpret_cast<const f4 *>(QKt + ti * 256 + m * 16 + 4 * g);
            }

        E *ap = apair + vu * (NPAIR * 64 * 8) + lane * 8;
        E *qp = qpair + vu * (NPAIR * 64 * 8) + lane * 8;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float eta = __expf((float)(Glast - Gs[16 * r + m]));
#pragma unroll
            for (int qq = 0; qq <= r / 2; ++qq) {
                f4 ev[2], ov[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int kb = 2 * qq + h;
                    ev[h] = f4{0, 0, 0, 0};
                    ov[h] = f4{0, 0, 0, 0};
                    if (kb <= r) {
                        const int ti = tri_index(r, kb);
                        const f4 bcol = *reinterpret_cast<const f4 *>(Bs + 16 * kb + 4 * g);
                        const f4 x4 = *reinterpret_cast<const f4 *>(Xw + ti * 256 + m * 16 + 4 * g);
                        ev[h] = eta * x4 * bcol;
                        f4 acc = {0, 0, 0, 0};
#pragma unroll
                        for (int mb = kb; mb <= r; ++mb)
                            acc = mma<F32>::block(acc, mma<F32>::from_f4(xt[tri_index(mb, kb)]),
                                                  mma<F32>::from_f4(aq[tri_index(r, mb)]));
                        ov[h] = acc * bcol;
                    }
                }
                const int p = pair_index(r, qq);
                *reinterpret_cast<V4 *>(ap + p * 512) = mma<F32>::from_f4(ev[0]);
                *reinterpret_cast<V4 *>(ap + p * 512 + 4) = mma<F32>::from_f4(ev[1]);
                *reinterpret_cast<V4 *>(qp + p * 512) = mma<F32>::from_f4(ov[0]);
                *reinterpret_cast<V4 *>(qp + p * 512 + 4) = mma<F32>::from_f4(ov[1]);
            }
        }
        wave_lds_sync();
    }
    __syncthreads();  // every wave is done with this unit's LDS before the next unit's images
    }
}

template <bool F32, typename TIn, int DK>
static hipError_t launch_chunk_local_t(const PrefillArgs &p, const PrefillWorkspace &ws, hipStream_t s) {
    typedef typename mma<F32>::E E;
    const int NC = (p.T + C - 1) / C;
    const int units = p.B * p.Hk * NC;
    // Resident work-groups walking the units (persistent), while that gives each
    // at most four units; beyond, one work-group per unit.  Measured: persistent
    // is faster at two units per work-group (30.5 against 33.5 us at T = 4096)
    // and slower from eight (107.8 against 103.5 us at T = 16384; 813 against
    // 757 us at two sequences of 65536 tokens).  The persistent loop's wait for
    // its own workspace stores (loads and stores share one counter) is not the
    // reason: an instance with a static value-head count, whose loop waits for
    // the loads alone, measured the same.
    int dev = 0, cus = 0, per_cu = 0;
    unsigned grid = (unsigned)units;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chunk_local_kernel<F32, TIn, DK>, 256, 0) == hipSuccess &&
        cus > 0 && per_cu > 0 && (long long)cus * per_cu < units && units <= 4LL * cus * per_cu)
        grid = (unsigned)(cus * per_cu);
    hipLaunchKernelGGL((chunk_local_kernel<F32, TIn, DK>), dim3(grid), dim3(256), 0, s, p.B, p.T,
                       p.Hk, p.Hv, NC, p.scale, (const TIn *)p.q, (const TIn *)p.k, p.a, p.b, p.A_log, p.dt_bias,
                       ws.tok, (E *)ws.apair, (E *)ws.qpair, (E *)ws.qimg, (E *)ws.kimg, (E *)ws.timg);
    return hipGetLastError();
}

hipError_t launch_chunk_local(const PrefillArgs &p, const PrefillWorkspace &ws, hipStream_t s) {
    if (p.f32) return p.Dk == 128 ? launch_chunk_local_t<true, float, 128>(p, ws, s)
                                   : launch_chunk_local_t<true, float, 64>(p, ws, s);
    return p.Dk == 128 ? launch_chunk_local_t<false, bf16_t, 128>(p, ws, s)
                       : launch_chunk_local_t<false, bf16_t, 64>(p, ws, s);
}

}  // namespace gdn
