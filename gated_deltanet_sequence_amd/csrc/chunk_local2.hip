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
//   - a diagonal tile: four dyadic levels (blocks of 16, 8, 4, 2 tokens); a
//     pair i < t belongs to the level whose block has i in its first and t in
//     its second half, with the first token of that half as reference: one
//     product per level, each lane a row or a column of it;
//   - the diagonal of A_qk carries no decay: q_t . k_t.
// G is kept in log2 units so that every decay factor is one exp2.  One
// work-group of 4 waves per (sequence, value head, chunk), 80 KB of LDS (two
// work-groups per compute unit).
#include "prefill_common.h"

namespace gdn {

size_t gdn2_workspace_layout(int B, int T, int Hv, int Dk, int Dv, bool f32, void *base, Gdn2Workspace *ws) {
    const size_t NC = (size_t)(T + C - 1) / C;
    const size_t vunits = (size_t)B * Hv * NC;
    const size_t esz = f32 ? 4 : 2;
    size_t off = 0;
    const size_t oE = off;  off = align256(off + vunits * C * Dk * esz);
    const size_t oKh = off; off = align256(off + vunits * C * Dk * esz);
    const size_t oQ = off;  off = align256(off + vunits * C * Dk * esz);
    const size_t oKt = off; off = align256(off + (f32 ? vunits * C * Dk * esz : 0));
    const size_t oA = off;  off = align256(off + vunits * NPAIR * 64 * 8 * esz);
    const size_t oAq = off; off = align256(off + vunits * NPAIR * 64 * 8 * esz);
    const size_t oG = off;  off = align256(off + vunits * Dk * 4);
    // Z = sigmoid(write) v: float32 only (the bfloat16 scan forms it from v and write)
    const size_t oZ = off;  off = align256(off + (f32 ? (size_t)B * T * Hv * Dv * esz : 0));
    if (ws) {
        char *p = (char *)base;
        ws->eimg = p + oE;
        ws->khimg = p + oKh;
        ws->qimg = p + oQ;
        ws->khtimg = f32 ? p + oKt : nullptr;
        ws->apair = p + oA;
        ws->qpair = p + oAq;
        ws->gc = (float *)(p + oG);
        ws->z = f32 ? p + oZ : nullptr;
        ws->bytes = off;
    }
    return off;
}

template <int DK>
struct Cl2Cfg {
    static constexpr int NT = 512;                     // threads per work-group (8 waves)
    static constexpr int NKQ = DK / 32;                // 32-deep contraction steps over the key channels
    static constexpr int NP = NT / DK, LEN = C / NP;   // prefix-sum parts per channel, tokens per part
    // LDS: G (float) and e, k, q (float16) as [C][DK] row-major with the
    // 16-byte pieces of each row XOR-swizzled by the row (no padding): 80 KB
    // at DK = 128, so two work-groups share a compute unit.
    static constexpr int LDS = C * DK * 4 + 3 * C * DK * 2;
    static_assert(3 * C * DK * 2 >= 2 * 10 * 256 * 4, "M and A_qk tiles reuse the e/k/q space");
    static_assert(C * DK * 4 >= 10 * 256 * 4, "the inverse's blocks reuse the G space");
};

// element (r, c) of a swizzled [C][DK] float / float16 array
template <int DK> __device__ __forceinline__ int gsw(int r, int c) {
    return r * DK + ((((c >> 2) ^ r) & (DK / 4 - 1)) << 2) + (c & 3);
}
template <int DK> __device__ __forceinline__ int hsw(int r, int c) {
    return r * DK + ((((c >> 3) ^ r) & (DK / 8 - 1)) << 3) + (c & 7);
}
// 8 consecutive channels c .. c+7 (c a multiple of 8) of row r
template <int DK> __device__ __forceinline__ void ldg8(const float *G, int r, int c, float (&x)[8]) {
    const f4 a = *reinterpret_cast<const f4 *>(G + gsw<DK>(r, c)), b = *reinterpret_cast<const f4 *>(G + gsw<DK>(r, c + 4));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[j] = a[j];
        x[4 + j] = b[j];
    }
}
template <int DK> __device__ __forceinline__ h8 ldh8(const _Float16 *X, int r, int c) {
    return *reinterpret_cast<const h8 *>(X + hsw<DK>(r, c));
}

// x (float16) times f (float32) as a float16 operand.  Written as an fma with a
// zero addend, which the compiler maps to v_fma_mix (the float16 input is
// converted inside the instruction); kept out of inline assembly, whose
// results the compiler's hazard checks do not see (a matrix-core product still
// reading an accumulator register it would overwrite).
__device__ __forceinline__ h8 mul_mix(h8 x, const float (&f)[8]) {
    h8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (_Float16)__builtin_fmaf((float)x[j], f[j], 0.f);
    return r;
}
// value of lane (4 (lane / 4) + P[lane % 4]) of x (a DPP quad permutation)
template <int CTRL> __device__ __forceinline__ float quad_perm(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

template <int DK, int DV>
__global__ __launch_bounds__(512, 4) void chunk_local2_kernel(
    int T, int Hk, int Hv, int NC, float scale, const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
    const bf16_t *__restrict__ a, const bf16_t *__restrict__ erase, const float *__restrict__ A_log,
    _Float16 *__restrict__ eimg,
    _Float16 *__restrict__ khimg, _Float16 *__restrict__ qimg, _Float16 *__restrict__ apair,
    _Float16 *__restrict__ qpair, float *__restrict__ gc) {
    typedef Cl2Cfg<DK> CF;
    constexpr int NKQ = CF::NKQ;
    __shared__ __attribute__((aligned(16))) char smem[CF::LDS];
    float *Gl = reinterpret_cast<float *>(smem);  // G in log2 units; later the inverse's blocks
    _Float16 *El = reinterpret_cast<_Float16 *>(smem + C * DK * 4), *Kl = El + C * DK, *Ql = Kl + C * DK;
    float *Ms = reinterpret_cast<float *>(El), *Qs = Ms + 10 * 256;  // lower 16x16 tiles of M, A_qk (after the tiles)

    const int u = blockIdx.x;
    const int n = u % NC, hv = (u / NC) % Hv, bb = u / (NC * Hv), hk = hv / (Hv / Hk);
    const int t0 = n * C;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t vu = ((size_t)bb * Hv + hv) * NC + n;
    constexpr float LOG2E = 1.4426950408889634f;

    // ---- 1. gates and key-side operands of the chunk into LDS (zero past T)
    //         (z = sigmoid(write) v is formed by the scan's state waves).  Every
    //         load of the phase is issued before any arithmetic; a thread sees
    //         the same 8 channels in each of its rows (512 is a multiple of
    //         DK / 8), so their decay rates exp(A_log) are loaded once.  g is
    //         kept in log2 units (g log2 e) so that every decay is one exp2.
    constexpr int NT = CF::NT, PK = C * (DK / 8) / NT;
    const int c8k = (tid % (DK / 8)) * 8;
    u16x8 rq[PK], rk[PK], ra[PK], re[PK];
    f4 Alo, Ahi;
    ld8(A_log, (size_t)hv * DK + c8k, Alo, Ahi);
#pragma unroll
    for (int it = 0; it < PK; ++it) {
        const int t = t0 + (tid + NT * it) / (DK / 8);
        rq[it] = rk[it] = ra[it] = re[it] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        if (t < T) {
            const size_t kq = (((size_t)bb * T + t) * Hk + hk) * DK + c8k;
            const size_t ka = (((size_t)bb * T + t) * Hv + hv) * DK + c8k;
            rq[it] = *reinterpret_cast<const u16x8 *>(reinterpret_cast<const uint16_t *>(q) + kq);
            rk[it] = *reinterpret_cast<const u16x8 *>(reinterpret_cast<const uint16_t *>(k) + kq);
            ra[it] = *reinterpret_cast<const u16x8 *>(reinterpret_cast<const uint16_t *>(a) + ka);
            re[it] = *reinterpret_cast<const u16x8 *>(reinterpret_cast<const uint16_t *>(erase) + ka);
        }
    }
    float rate[8];  // exp(A_log) log2 e
#pragma unroll
    for (int j = 0; j < 8; ++j) rate[j] = exp_fast(j < 4 ? Alo[j] : Ahi[j - 4]) * LOG2E;
#pragma unroll
    for (int it = 0; it < PK; ++it) {
        const int r = (tid + NT * it) / (DK / 8), t = t0 + r;
        float gv[8];
        h8 eh, kh, qh;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float kv = bf16_to_f32(rk[it][j]);
            gv[j] = t < T ? -rate[j] * softplus_fast(bf16_to_f32(ra[it][j])) : 0.f;
            eh[j] = (_Float16)(sigmoid_fast(bf16_to_f32(re[it][j])) * kv);
            kh[j] = (_Float16)kv;
            qh[j] = (_Float16)(scale * bf16_to_f32(rq[it][j]));
        }
        *reinterpret_cast<f4 *>(Gl + gsw<DK>(r, c8k)) = f4{gv[0], gv[1], gv[2], gv[3]};
        *reinterpret_cast<f4 *>(Gl + gsw<DK>(r, c8k + 4)) = f4{gv[4], gv[5], gv[6], gv[7]};
        *reinterpret_cast<h8 *>(El + hsw<DK>(r, c8k)) = eh;
        *reinterpret_cast<h8 *>(Kl + hsw<DK>(r, c8k)) = kh;
        *reinterpret_cast<h8 *>(Ql + hsw<DK>(r, c8k)) = qh;
    }
    __syncthreads();

    // ---- 2. G: inclusive prefix of g over the chunk's tokens, per channel, in
    //         NP parts of LEN tokens; a part adds the local totals of the parts
    //         before it (read from their last rows between two barriers)
    {
        const int c = tid % DK, part = tid / DK;
        float x[CF::LEN];
#pragma unroll
        for (int j = 0; j < CF::LEN; ++j) x[j] = Gl[gsw<DK>(part * CF::LEN + j, c)];
#pragma unroll
        for (int j = 1; j < CF::LEN; ++j) x[j] += x[j - 1];
        Gl[gsw<DK>(part * CF::LEN + CF::LEN - 1, c)] = x[CF::LEN - 1];
        __syncthreads();
        float off = 0.f;
        for (int p = 0; p < part; ++p) off += Gl[gsw<DK>(p * CF::LEN + CF::LEN - 1, c)];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < CF::LEN; ++j) Gl[gsw<DK>(part * CF::LEN + j, c)] = x[j] + off;
    }
    __syncthreads();

    // ---- 3. the scan's operand images (Et, Kh, Qt) and e^{G_C}.  A thread
    //         writes physical 8-group P of image row r, which holds logical
    //         columns lc .. lc+3 and lc+16 .. lc+19 (perm_col), lc = 32(P/4) + 4(P%4)
#pragma unroll
    for (int it = 0; it < PK; ++it) {
        const int idx = tid + NT * it, r = idx / (DK / 8), P = idx % (DK / 8);
        const int lc = 32 * (P / 4) + 4 * (P % 4);
        h8 eo, ko, qo;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int c = lc + 16 * hh;
            const f4 gt = *reinterpret_cast<const f4 *>(Gl + gsw<DK>(r, c));
            const f4 gC = *reinterpret_cast<const f4 *>(Gl + gsw<DK>(C - 1, c));
            typedef _Float16 h4v __attribute__((ext_vector_type(4)));
            const h4v ev = *reinterpret_cast<const h4v *>(El + hsw<DK>(r, c));
            const h4v kv = *reinterpret_cast<const h4v *>(Kl + hsw<DK>(r, c));
            const h4v qv = *reinterpret_cast<const h4v *>(Ql + hsw<DK>(r, c));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float fe = __builtin_amdgcn_exp2f(gt[j]), fk = __builtin_amdgcn_exp2f(gC[j] - gt[j]);
                eo[4 * hh + j] = (_Float16)((float)ev[j] * fe);
                qo[4 * hh + j] = (_Float16)((float)qv[j] * fe);
                ko[4 * hh + j] = (_Float16)((float)kv[j] * fk);
            }
        }
        const size_t o = vu * C * DK + img_index<false>(r, DK, P * 8);
        *reinterpret_cast<h8 *>(eimg + o) = eo;
        *reinterpret_cast<h8 *>(khimg + o) = ko;
        *reinterpret_cast<h8 *>(qimg + o) = qo;
    }
    if (tid < DK) gc[vu * DK + tid] = __builtin_amdgcn_exp2f(Gl[gsw<DK>(C - 1, tid)]);

    // ---- 4. tiles of M and A_qk below the diagonal (rows 16I, columns 16J,
    //         I > J): reference token 16I.  A = k e^{G_ref - G} (column rows),
    //         B = e e^{G - G_ref} or q e^{G - G_ref} (row rows): the accumulator
    //         holds row 16I + m, columns 16J + 4g .. +3.  A wave takes whole row
    //         tiles, so the row side (its factors and both B operands) is formed
    //         once for its tiles: wave 0 (1,0) (it alone runs the inverse
    //         afterwards), wave 1 (2,0) (2,1), wave 2 (3,0) (3,1), wave 3 (3,2).
    //         The results stay in registers until the e/k/q space is free.
    const int wo = w - 4;  // waves 4..7 take the tiles below the diagonal, waves 0..3 the diagonal ones
    const int oI = wo == 0 ? 1 : wo == 1 ? 2 : 3, oJ0 = wo == 3 ? 2 : 0, onj = (wo == 1 || wo == 2) ? 2 : 1;
    f4 oM[2], oQ[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) oM[h] = oQ[h] = f4{0, 0, 0, 0};
    if (w >= 4) {
        const int ref = 16 * oI, tr = 16 * oI + m;
#pragma unroll
        for (int kq = 0; kq < NKQ; ++kq) {
            const int c = 32 * kq + 8 * g;
            float gt[8], gr[8], fl[8];
            ldg8<DK>(Gl, tr, c, gt);
            ldg8<DK>(Gl, ref, c, gr);
#pragma unroll
            for (int j = 0; j < 8; ++j) fl[j] = __builtin_amdgcn_exp2f(gt[j] - gr[j]);
            const h8 be = mul_mix(ldh8<DK>(El, tr, c), fl), bq = mul_mix(ldh8<DK>(Ql, tr, c), fl);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (h < onj) {
                    const int ir = 16 * (oJ0 + h) + m;
                    float gi[8], fr[8];
                    ldg8<DK>(Gl, ir, c, gi);
#pragma unroll
                    for (int j = 0; j < 8; ++j) fr[j] = __builtin_amdgcn_exp2f(gr[j] - gi[j]);
                    const h8 rk8 = mul_mix(ldh8<DK>(Kl, ir, c), fr);
                    oM[h] = mfma_f16_k32(rk8, be, oM[h]);
                    oQ[h] = mfma_f16_k32(rk8, bq, oQ[h]);
                }
            }
        }
    }

    // ---- 5. diagonal tile I = w, token r0 + m in lane (g, m).  Every pair
    //         i < t of the tile is split at the coarsest of four dyadic levels
    //         where i and t fall into the two halves of one block (block sizes
    //         16, 8, 4, 2): at that level the reference is the first token of
    //         the block's second half, every lane is a column (first half,
    //         factor e^{G_ref - G_i}) or a row (second half, e^{G_t - G_ref}),
    //         both e^{-|G - G_ref|}, one exp2 per lane and channel and level.
    //         One product per level and matrix; each level's accumulator keeps
    //         only its own pairs.  The diagonal of A_qk (no decay) is q.k.
    f4 dM = {0, 0, 0, 0}, dQ = {0, 0, 0, 0};
    if (w < 4) {
        const int r0 = 16 * w, t = r0 + m;
        f4 aM[4], aQ[4];
#pragma unroll
        for (int l = 0; l < 4; ++l) aM[l] = aQ[l] = f4{0, 0, 0, 0};
        float dq = 0.f;
#pragma unroll
        for (int kq = 0; kq < NKQ; ++kq) {
            const int c = 32 * kq + 8 * g;
            float gt[8], g0[8], g1[8];
            ldg8<DK>(Gl, t, c, gt);
            ldg8<DK>(Gl, r0 + 8, c, g0);             // level 0: reference 8
            ldg8<DK>(Gl, r0 + (m & 8) + 4, c, g1);   // level 1: reference 4 or 12
            const h8 et = ldh8<DK>(El, t, c), qt = ldh8<DK>(Ql, t, c), kt = ldh8<DK>(Kl, t, c);
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                typedef _Float16 h2v __attribute__((ext_vector_type(2)));
                dq = __builtin_amdgcn_fdot2(h2v{qt[j], qt[j + 1]}, h2v{kt[j], kt[j + 1]}, dq, false);
            }
#pragma unroll
            for (int l = 0; l < 4; ++l) {
                float f[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    // level 2: reference lane 2 of the quad; level 3: lane 1 or 3
                    const float gr = l == 0 ? g0[j] : l == 1 ? g1[j] : l == 2 ? quad_perm<0xAA>(gt[j]) : quad_perm<0xF5>(gt[j]);
                    f[j] = __builtin_amdgcn_exp2f(-fabsf(gt[j] - gr));
                }
                const h8 A = mul_mix(kt, f);
                aM[l] = mfma_f16_k32(A, mul_mix(et, f), aM[l]);
                aQ[l] = mfma_f16_k32(A, mul_mix(qt, f), aQ[l]);
            }
        }
        // lane holds pairs (i = 4g + s, t = m)
#pragma unroll
        for (int l = 0; l < 4; ++l) {
            const int b = 16 >> l, hb = b >> 1;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int i = 4 * g + s;
                const bool mine = (i / b == m / b) && (i % b < hb) && (m % b >= hb);
                dM[s] += mine ? aM[l][s] : 0.f;
                dQ[s] += mine ? aQ[l][s] : 0.f;
            }
        }
        dq += __shfl_xor(dq, 16, 64);
        dq += __shfl_xor(dq, 32, 64);
#pragma unroll
        for (int s = 0; s < 4; ++s)
            if (4 * g + s == m) dQ[s] += dq;
    }
    __syncthreads();  // G, e, k, q are dead: the tiles take their space
    if (w >= 4) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (h < onj) {
                *reinterpret_cast<f4 *>(Ms + tri_index(oI, oJ0 + h) * 256 + m * 16 + 4 * g) = oM[h];
                *reinterpret_cast<f4 *>(Qs + tri_index(oI, oJ0 + h) * 256 + m * 16 + 4 * g) = oQ[h];
            }
        }
    } else {
        *reinterpret_cast<f4 *>(Ms + tri_index(w, w) * 256 + m * 16 + 4 * g) = dM;
        *reinterpret_cast<f4 *>(Qs + tri_index(w, w) * 256 + m * 16 + 4 * g) = dQ;
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
    {   // lane (block bq, column c): column c of the block's inverse, x[r] = delta_rc to
        // start; L[r][j] from lane j of the same 16-lane row by a DPP row broadcast
        const int bq = lane >> 4, c = lane & 15;
        const float *Lb = Ms + tri_index(bq, bq) * 256;
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
    hipLaunchKernelGGL((chunk_local2_kernel<DK, DV>), dim3(units), dim3(Cl2Cfg<DK>::NT), 0, s, p.T, p.Hk, p.Hv, NC, p.scale,
                       (const bf16_t *)p.q, (const bf16_t *)p.k, (const bf16_t *)p.a,
                       (const bf16_t *)p.erase, p.A_log, (_Float16 *)ws.eimg,
                       (_Float16 *)ws.khimg, (_Float16 *)ws.qimg, (_Float16 *)ws.apair, (_Float16 *)ws.qpair,
                       ws.gc);
    return hipGetLastError();
}

hipError_t launch_chunk_local2(const Gdn2Args &p, const Gdn2Workspace &ws, hipStream_t s) {
    if (p.f32) return launch_chunk_local2_f32(p, ws, s);
    if (p.Dk == 128 && p.Dv == 128) return launch_cl2_t<128, 128>(p, ws, s);
    if (p.Dk == 128 && p.Dv == 64) return launch_cl2_t<128, 64>(p, ws, s);
    if (p.Dk == 64 && p.Dv == 128) return launch_cl2_t<64, 128>(p, ws, s);
    if (p.Dk == 64 && p.Dv == 64) return launch_cl2_t<64, 64>(p, ws, s);
    return hipErrorInvalidValue;
}

}  // namespace gdn
