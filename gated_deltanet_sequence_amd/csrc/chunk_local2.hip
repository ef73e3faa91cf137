// chunk_local2.hip -- chunk-local auxiliaries of the Gated DeltaNet-2 chunked
// prefill (channel-wise decay, erase and write gates), bfloat16 inputs with
// float16 matrix-core operands.
//
// Recurrence (zhichai.net "Gated DeltaNet-2" digest, sections on the decoupled
// erase/write update and "高效训练：WY 算法依然成立"): per token,
//   Sbar = diag(D_t) S,  D_t = e^{g_t} (per key channel),
//   S    = Sbar + k_t (z_t - Sbar^T e_t)^T,  e_t = b_t (.) k_t,  z_t = w_t (.) v_t,
//   o_t  = scale S^T q_t.
// With G_t the in-chunk inclusive prefix of g (a vector over key channels) and
// chunk-start state S0, unrolling the chunk gives
//   U   = A (Z - Et S0),        A = (I + M)^{-1},
//   M   = strictly-lower( sum_c e_t[c] k_i[c] e^{G_t[c] - G_i[c]} ),
//   O   = Qt S0 + A_qk U,       A_qk = lower-incl-diag( scale sum_c q_t[c] k_i[c] e^{G_t[c] - G_i[c]} ),
//   S'  = diag(e^{G_C}) S0 + Kh^T U,
// where Et = e (.) e^{G}, Qt = scale q (.) e^{G}, Kh = k (.) e^{G_C - G} (every
// factor <= 1).  The scan applies U = A R' and O = Qt S0 + (A_qk A) R' to the
// residual R' = Z - Et S0.
//
// M and A_qk need a decay ratio per (row, column, channel).  No factor may
// exceed 1 (per-token decays reach e^-50), so each product is split at a
// reference token between the row and the column:
//   - a 16x16 tile below the diagonal (rows I > columns J): reference 16I, one
//     float16 matrix-core product of (k e^{G_ref - G}) and (e e^{G - G_ref});
//   - a diagonal tile: three products with references at 4-token steps, each
//     taking the columns of one 4-token sub-block and every later row;
//   - entries inside a 4-token diagonal sub-block: elementwise in float32.
// One work-group of 4 waves per (sequence, value head, chunk).
#include "prefill_common.h"

namespace gdn {

size_t gdn2_workspace_layout(int B, int T, int Hv, int Dk, int Dv, void *base, Gdn2Workspace *ws) {
    const size_t NC = (size_t)(T + C - 1) / C;
    const size_t vunits = (size_t)B * Hv * NC;
    size_t off = 0;
    const size_t oE = off;  off = align256(off + vunits * C * Dk * 2);
    const size_t oKh = off; off = align256(off + vunits * C * Dk * 2);
    const size_t oQ = off;  off = align256(off + vunits * C * Dk * 2);
    const size_t oA = off;  off = align256(off + vunits * NPAIR * 64 * 8 * 2);
    const size_t oAq = off; off = align256(off + vunits * NPAIR * 64 * 8 * 2);
    const size_t oG = off;  off = align256(off + vunits * Dk * 4);
    const size_t oZ = off;  off = align256(off + (size_t)B * T * Hv * Dv * 2);
    if (ws) {
        char *p = (char *)base;
        ws->eimg = p + oE;
        ws->khimg = p + oKh;
        ws->qimg = p + oQ;
        ws->apair = p + oA;
        ws->qpair = p + oAq;
        ws->gc = (float *)(p + oG);
        ws->z = p + oZ;
        ws->bytes = off;
    }
    return off;
}

template <int DK>
struct Cl2Cfg {
    static constexpr int GS = DK + 4;  // float row stride of G in LDS (16-byte pad: rows land on distinct banks)
    static constexpr int HS = DK + 8;  // half row stride of e, k, q in LDS
    static constexpr int NP = 256 / DK, LEN = C / NP;  // prefix-sum parts per channel, tokens per part
};

__device__ __forceinline__ void ld8h(const _Float16 *p, float (&x)[8]) {
    const h8 v = *reinterpret_cast<const h8 *>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = (float)v[j];
}
__device__ __forceinline__ void ld8f(const float *p, float (&x)[8]) {
    const f4 a = *reinterpret_cast<const f4 *>(p), b = *reinterpret_cast<const f4 *>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[j] = a[j];
        x[4 + j] = b[j];
    }
}

template <int DK, int DV>
__global__ __launch_bounds__(256) void chunk_local2_kernel(
    int T, int Hk, int Hv, int NC, float scale, const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
    const bf16_t *__restrict__ v, const bf16_t *__restrict__ a, const bf16_t *__restrict__ erase,
    const bf16_t *__restrict__ write, const float *__restrict__ A_log, _Float16 *__restrict__ eimg,
    _Float16 *__restrict__ khimg, _Float16 *__restrict__ qimg, _Float16 *__restrict__ apair,
    _Float16 *__restrict__ qpair, float *__restrict__ gc, _Float16 *__restrict__ z) {
    typedef Cl2Cfg<DK> CF;
    constexpr int GS = CF::GS, HS = CF::HS;
    __shared__ __attribute__((aligned(16))) float Gl[C * GS];  // g, then G; the inverse's scratch at the end
    __shared__ __attribute__((aligned(16))) _Float16 El[C * HS], Kl[C * HS], Ql[C * HS];
    __shared__ __attribute__((aligned(16))) float Ms[10 * 256], Qs[10 * 256];  // lower 16x16 tiles of M, A_qk
    __shared__ float tot[CF::NP][DK];

    const int u = blockIdx.x;
    const int n = u % NC, hv = (u / NC) % Hv, bb = u / (NC * Hv), hk = hv / (Hv / Hk);
    const int t0 = n * C;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t vu = ((size_t)bb * Hv + hv) * NC + n;

    // ---- 1. gates and key-side operands of the chunk into LDS (zero past T);
    //         z = sigmoid(write) v to the workspace
    constexpr int PK = C * (DK / 8) / 256, PV = C * (DV / 8) / 256;
#pragma unroll
    for (int it = 0; it < PK; ++it) {
        const int idx = tid + 256 * it, r = idx / (DK / 8), c8 = (idx % (DK / 8)) * 8, t = t0 + r;
        f4 q0 = {0, 0, 0, 0}, q1 = q0, k0 = q0, k1 = q0, a0 = q0, a1 = q0, e0 = q0, e1 = q0;
        if (t < T) {
            const size_t kq = (((size_t)bb * T + t) * Hk + hk) * DK + c8;
            const size_t ka = (((size_t)bb * T + t) * Hv + hv) * DK + c8;
            ld8(q, kq, q0, q1);
            ld8(k, kq, k0, k1);
            ld8(a, ka, a0, a1);
            ld8(erase, ka, e0, e1);
        }
        float gv[8];
        h8 eh, kh, qh;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float av = j < 4 ? a0[j] : a1[j - 4], ev = j < 4 ? e0[j] : e1[j - 4];
            const float kv = j < 4 ? k0[j] : k1[j - 4], qv = j < 4 ? q0[j] : q1[j - 4];
            gv[j] = t < T ? -exp_fast(A_log[(size_t)hv * DK + c8 + j]) * softplus_fast(av) : 0.f;
            eh[j] = (_Float16)(sigmoid_fast(ev) * kv);
            kh[j] = (_Float16)kv;
            qh[j] = (_Float16)(scale * qv);
        }
        *reinterpret_cast<f4 *>(Gl + r * GS + c8) = f4{gv[0], gv[1], gv[2], gv[3]};
        *reinterpret_cast<f4 *>(Gl + r * GS + c8 + 4) = f4{gv[4], gv[5], gv[6], gv[7]};
        *reinterpret_cast<h8 *>(El + r * HS + c8) = eh;
        *reinterpret_cast<h8 *>(Kl + r * HS + c8) = kh;
        *reinterpret_cast<h8 *>(Ql + r * HS + c8) = qh;
    }
#pragma unroll
    for (int it = 0; it < PV; ++it) {
        const int idx = tid + 256 * it, r = idx / (DV / 8), c8 = (idx % (DV / 8)) * 8, t = t0 + r;
        if (t < T) {
            const size_t kv = (((size_t)bb * T + t) * Hv + hv) * DV + c8;
            f4 v0, v1, w0, w1;
            ld8(v, kv, v0, v1);
            ld8(write, kv, w0, w1);
            h8 zh;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                zh[j] = (_Float16)(sigmoid_fast(w0[j]) * v0[j]);
                zh[4 + j] = (_Float16)(sigmoid_fast(w1[j]) * v1[j]);
            }
            *reinterpret_cast<h8 *>(z + kv) = zh;
        }
    }
    __syncthreads();

    // ---- 2. G: inclusive prefix of g over the chunk's tokens, per channel
    {
        const int c = tid % DK, part = tid / DK;
        float x[CF::LEN];
#pragma unroll
        for (int j = 0; j < CF::LEN; ++j) x[j] = Gl[(part * CF::LEN + j) * GS + c];
#pragma unroll
        for (int j = 1; j < CF::LEN; ++j) x[j] += x[j - 1];
        tot[part][c] = x[CF::LEN - 1];
        __syncthreads();
        float off = 0.f;
        for (int p = 0; p < part; ++p) off += tot[p][c];
#pragma unroll
        for (int j = 0; j < CF::LEN; ++j) Gl[(part * CF::LEN + j) * GS + c] = x[j] + off;
    }
    __syncthreads();

    // ---- 3. the scan's operand images (Et, Kh, Qt) and e^{G_C}.  A thread
    //         writes physical 8-group P of image row r, which holds logical
    //         columns lc .. lc+3 and lc+16 .. lc+19 (perm_col), lc = 32(P/4) + 4(P%4)
#pragma unroll
    for (int it = 0; it < PK; ++it) {
        const int idx = tid + 256 * it, r = idx / (DK / 8), P = idx % (DK / 8);
        const int lc = 32 * (P / 4) + 4 * (P % 4);
        h8 eo, ko, qo;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int c = lc + 16 * hh;
            const f4 gt = *reinterpret_cast<const f4 *>(Gl + r * GS + c);
            const f4 gC = *reinterpret_cast<const f4 *>(Gl + (C - 1) * GS + c);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float fe = exp_fast(gt[j]), fk = exp_fast(gC[j] - gt[j]);
                eo[4 * hh + j] = (_Float16)((float)El[r * HS + c + j] * fe);
                qo[4 * hh + j] = (_Float16)((float)Ql[r * HS + c + j] * fe);
                ko[4 * hh + j] = (_Float16)((float)Kl[r * HS + c + j] * fk);
            }
        }
        const size_t o = vu * C * DK + img_index<false>(r, DK, P * 8);
        *reinterpret_cast<h8 *>(eimg + o) = eo;
        *reinterpret_cast<h8 *>(khimg + o) = ko;
        *reinterpret_cast<h8 *>(qimg + o) = qo;
    }
    if (tid < DK) gc[vu * DK + tid] = exp_fast(Gl[(C - 1) * GS + tid]);

    // ---- 4. tiles of M and A_qk below the diagonal (rows 16I, columns 16J,
    //         I > J): reference token 16I.  A = k e^{G_ref - G} (column rows),
    //         B = e e^{G - G_ref} or q e^{G - G_ref} (row rows): the accumulator
    //         holds row 16I + m, columns 16J + 4g .. +3 (the operand layout the
    //         inverse reads)
    {
        constexpr int TI[6] = {1, 2, 2, 3, 3, 3}, TJ[6] = {0, 0, 1, 0, 1, 2};
        for (int p = w; p < 6; p += 4) {
            const int I = TI[p], J = TJ[p], ref = 16 * I, tr = 16 * I + m, ir = 16 * J + m;
            f4 accM = {0, 0, 0, 0}, accQ = accM;
#pragma unroll
            for (int kq = 0; kq < DK / 32; ++kq) {
                const int c = 32 * kq + 8 * g;
                float gt[8], gr[8], gi[8], et[8], qt[8], ki[8];
                ld8f(Gl + tr * GS + c, gt);
                ld8f(Gl + ref * GS + c, gr);
                ld8f(Gl + ir * GS + c, gi);
                ld8h(El + tr * HS + c, et);
                ld8h(Ql + tr * HS + c, qt);
                ld8h(Kl + ir * HS + c, ki);
                h8 le, lq, rk;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float fl = exp_fast(gt[j] - gr[j]), fr = exp_fast(gr[j] - gi[j]);
                    le[j] = (_Float16)(et[j] * fl);
                    lq[j] = (_Float16)(qt[j] * fl);
                    rk[j] = (_Float16)(ki[j] * fr);
                }
                accM = mfma_f16_k32(rk, le, accM);
                accQ = mfma_f16_k32(rk, lq, accQ);
            }
            *reinterpret_cast<f4 *>(Ms + tri_index(I, J) * 256 + m * 16 + 4 * g) = accM;
            *reinterpret_cast<f4 *>(Qs + tri_index(I, J) * 256 + m * 16 + 4 * g) = accQ;
        }
    }

    // ---- 5. diagonal tile I = w
    {
        const int I = w, r0 = 16 * I, t = r0 + m;
        f4 accM = {0, 0, 0, 0}, accQ = accM;
        // (a) columns in an earlier 4-token sub-block than the row: reference
        //     token r0 + 4s takes the columns of sub-block s-1 and rows >= r0 + 4s
        for (int s = 1; s < 4; ++s) {
            const int ref = r0 + 4 * s;
            const bool lrow = m >= 4 * s, rrow = m >= 4 * s - 4 && m < 4 * s;
#pragma unroll
            for (int kq = 0; kq < DK / 32; ++kq) {
                const int c = 32 * kq + 8 * g;
                float gt[8], gr[8], et[8], qt[8], kt[8];
                ld8f(Gl + t * GS + c, gt);
                ld8f(Gl + ref * GS + c, gr);
                ld8h(El + t * HS + c, et);
                ld8h(Ql + t * HS + c, qt);
                ld8h(Kl + t * HS + c, kt);
                h8 le, lq, rk;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    // each factor is taken only where its exponent is <= 0
                    const float fl = exp_fast(fminf(gt[j] - gr[j], 0.f)), fr = exp_fast(fminf(gr[j] - gt[j], 0.f));
                    le[j] = lrow ? (_Float16)(et[j] * fl) : (_Float16)0.f;
                    lq[j] = lrow ? (_Float16)(qt[j] * fl) : (_Float16)0.f;
                    rk[j] = rrow ? (_Float16)(kt[j] * fr) : (_Float16)0.f;
                }
                accM = mfma_f16_k32(rk, le, accM);
                accQ = mfma_f16_k32(rk, lq, accQ);
            }
        }
        // (b) columns in the row's own 4-token sub-block, elementwise in
        //     float32: lane group g sums a quarter of the channels, then the
        //     four groups are added across lanes
        const int base = r0 + 4 * (m / 4);
        float pm[4] = {0, 0, 0, 0}, pq[4] = {0, 0, 0, 0};
        constexpr int NCH = DK / 4;
        for (int cc = 0; cc < NCH; cc += 8) {
            const int c = g * NCH + cc;
            float gt[8], et[8], qt[8];
            ld8f(Gl + t * GS + c, gt);
            ld8h(El + t * HS + c, et);
            ld8h(Ql + t * HS + c, qt);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int i = base + s;
                float gi[8], ki[8];
                ld8f(Gl + i * GS + c, gi);
                ld8h(Kl + i * HS + c, ki);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float f = exp_fast(fminf(gt[j] - gi[j], 0.f)) * ki[j];  // columns past the row are dropped below
                    pm[s] += et[j] * f;
                    pq[s] += qt[j] * f;
                }
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            pm[s] += __shfl_xor(pm[s], 16, 64);
            pm[s] += __shfl_xor(pm[s], 32, 64);
            pq[s] += __shfl_xor(pq[s], 16, 64);
            pq[s] += __shfl_xor(pq[s], 32, 64);
        }
        if (g == m / 4) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int i = base + s;
                accM[s] += i < t ? pm[s] : 0.f;
                accQ[s] += i <= t ? pq[s] : 0.f;
            }
        }
        *reinterpret_cast<f4 *>(Ms + tri_index(I, I) * 256 + m * 16 + 4 * g) = accM;
        *reinterpret_cast<f4 *>(Qs + tri_index(I, I) * 256 + m * 16 + 4 * g) = accQ;
    }
    __syncthreads();
    if (w != 0) return;

    // ---- 6. A = (I + M)^{-1} (wave 0): diagonal 16x16 blocks by forward
    //         substitution, off-diagonal blocks on the matrix cores
    float *Xw = Gl;  // G is dead: 10 blocks of X
    f4 Lf[10];
#pragma unroll
    for (int rb = 1; rb < 4; ++rb)
#pragma unroll
        for (int kb = 0; kb < rb; ++kb)
            Lf[tri_index(rb, kb)] = *reinterpret_cast<const f4 *>(Ms + tri_index(rb, kb) * 256 + m * 16 + 4 * g);
    {
        const int bq = lane >> 4, c = lane & 15;
        const float *Lb = Ms + tri_index(bq, bq) * 256;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s = (r == c) ? 1.f : 0.f;
#pragma unroll
            for (int jj = 0; jj < r; ++jj) s -= Lb[r * 16 + jj] * x[jj];
            x[r] = s;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) Xw[tri_index(bq, bq) * 256 + r * 16 + c] = x[r];
    }
    wave_lds_sync();
    f4 xt[10];  // blocks of A in accumulator layout: lane holds A[16i + 4g + s][16j + m]
    inverse_offdiag<false>(Xw, Lf, m, g, xt);
    wave_lds_sync();

    // ---- 7. operand fragments of A and of A_qk A (the latter from the matrix
    //         cores as (A_qk A)^T = A^T A_qk^T, whose accumulator is its
    //         operand layout)
    f4 aq[10];
#pragma unroll
    for (int ti = 0; ti < 10; ++ti) aq[ti] = *reinterpret_cast<const f4 *>(Qs + ti * 256 + m * 16 + 4 * g);
    _Float16 *ap = apair + vu * (NPAIR * 64 * 8) + lane * 8;
    _Float16 *qp = qpair + vu * (NPAIR * 64 * 8) + lane * 8;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int qq = 0; qq <= r / 2; ++qq) {
            f4 ev[2], ov[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int kb = 2 * qq + h;
                ev[h] = f4{0, 0, 0, 0};
                ov[h] = f4{0, 0, 0, 0};
                if (kb <= r) {
                    ev[h] = *reinterpret_cast<const f4 *>(Xw + tri_index(r, kb) * 256 + m * 16 + 4 * g);
                    f4 acc = {0, 0, 0, 0};
#pragma unroll
                    for (int mb = kb; mb <= r; ++mb)
                        acc = mma<false>::block(acc, to_h4(xt[tri_index(mb, kb)]), to_h4(aq[tri_index(r, mb)]));
                    ov[h] = acc;
                }
            }
            const int p = pair_index(r, qq);
            *reinterpret_cast<h4 *>(ap + p * 512) = to_h4(ev[0]);
            *reinterpret_cast<h4 *>(ap + p * 512 + 4) = to_h4(ev[1]);
            *reinterpret_cast<h4 *>(qp + p * 512) = to_h4(ov[0]);
            *reinterpret_cast<h4 *>(qp + p * 512 + 4) = to_h4(ov[1]);
        }
    }
}

template <int DK, int DV>
static hipError_t launch_cl2_t(const Gdn2Args &p, const Gdn2Workspace &ws, hipStream_t s) {
    const int NC = (p.T + C - 1) / C;
    const unsigned units = (unsigned)(p.B * p.Hv * NC);
    hipLaunchKernelGGL((chunk_local2_kernel<DK, DV>), dim3(units), dim3(256), 0, s, p.T, p.Hk, p.Hv, NC, p.scale,
                       (const bf16_t *)p.q, (const bf16_t *)p.k, (const bf16_t *)p.v, (const bf16_t *)p.a,
                       (const bf16_t *)p.erase, (const bf16_t *)p.write, p.A_log, (_Float16 *)ws.eimg,
                       (_Float16 *)ws.khimg, (_Float16 *)ws.qimg, (_Float16 *)ws.apair, (_Float16 *)ws.qpair,
                       ws.gc, (_Float16 *)ws.z);
    return hipGetLastError();
}

hipError_t launch_chunk_local2(const Gdn2Args &p, const Gdn2Workspace &ws, hipStream_t s) {
    if (p.Dk == 128 && p.Dv == 128) return launch_cl2_t<128, 128>(p, ws, s);
    if (p.Dk == 128 && p.Dv == 64) return launch_cl2_t<128, 64>(p, ws, s);
    if (p.Dk == 64 && p.Dv == 128) return launch_cl2_t<64, 128>(p, ws, s);
    if (p.Dk == 64 && p.Dv == 64) return launch_cl2_t<64, 64>(p, ws, s);
    return hipErrorInvalidValue;
}

}  // namespace gdn
