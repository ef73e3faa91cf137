// prefill_common.h -- definitions shared by the chunked-prefill kernels.
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
#pragma once

#include <utility>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

static constexpr int C = 64;      // chunk length
static constexpr int NPAIR = 6;   // operand fragments ("pairs") of a strictly-lower 64x64 matrix

// Pair fragments of a strictly-lower 64x64 matrix M: row tile r (16 rows)
// needs k-steps q = 0..r/2 (32 columns each); pair (r, q) holds, for lane
// l = 16 g + m, the 8 values M[16r+m][32q + 4g + i] and M[16r+m][32q + 16 + 4g + i]
// (i = 0..3), contiguous per lane.  pair_index numbers the pairs 0..5.
__host__ __device__ constexpr int pair_base(int r) { return r == 0 ? 0 : r == 1 ? 1 : r == 2 ? 2 : 4; }
__host__ __device__ constexpr int pair_index(int r, int q) { return pair_base(r) + q; }

// Column permutation used when staging a row-major operand in LDS for the
// float16 products: inside each 32-column block, logical column k goes to
// position 8*((k%16)/4) + 4*(k/16) + k%4, so the 8 values a lane contributes to
// one 16x16x32 step (k-blocks 4g..4g+3 and 16+4g..16+4g+3) are contiguous and
// come in one 16-byte LDS read.  The float32 products read 4 values per k-block,
// already contiguous: no permutation.
template <bool F32>
__host__ __device__ constexpr int perm_col(int k) {
    return F32 ? k : (k & ~31) | (((k & 15) >> 2) << 3) | (((k & 31) >> 4) << 2) | (k & 3);
}

// Tile images.  Q and K of a chunk ([64 tokens][d_k]) and, for float32
// operands, K^T ([d_k][64 tokens]) are kept as row-major tiles of the operand
// type, columns placed by perm_col
// and each row's 16-byte groups XOR-swizzled by a function of the row
// (img_swz): the 16 lanes that read the same group of 16 consecutive rows in
// one instruction then cover all 64 LDS banks (256 bytes), with no padding.
// The chunk-local kernel writes the images to the workspace in exactly this
// layout and the scan copies them byte for byte into LDS.
template <bool F32>
__host__ __device__ constexpr int img_epg() { return F32 ? 4 : 8; }  // elements per 16-byte group

// Group swizzle of image row `row` (LDS has 64 four-byte banks, 256 bytes).
// 256-byte float16 rows (16 groups) XOR the group with the low 4 bits of the
// row, rotated by two: ((row & 3) << 2) | ((row >> 2) & 3).  Being a bijection
// of row & 15, it keeps the operand reads of 16 consecutive rows (one group
// each) on 16 distinct groups; and the transposed reads of the state update
// -- 4 consecutive rows (row & 3 = 0..3) times 4 consecutive groups (the low
// two group bits) -- also land on 16 distinct groups, since the row's low
// bits go to the high group bits.  128-byte float16 rows hold two rows per
// 256 bytes: XOR with (row >> 1) & 7, the row parity picks the half.
// Float32 rows XOR with row & 7.
template <bool F32>
__host__ __device__ constexpr int img_swz(int row, int rowlen) {
    return F32 ? (row & 7) : rowlen >= 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((row >> 1) & 7);
}

template <bool F32>
__device__ __forceinline__ int img_index(int row, int rowlen, int phys) {
    constexpr int epg = img_epg<F32>();
    return row * rowlen + (((phys / epg) ^ img_swz<F32>(row, rowlen)) * epg) + phys % epg;
}

// Operand pair (two 16-deep k-blocks, logical columns 32kq .. 32kq+31) of image
// row R for lane group g.
template <bool F32>
__device__ __forceinline__ void img_pair(const typename mma<F32>::E *X, int rowlen, int R, int kq, int g,
                                         typename mma<F32>::V4 &a0, typename mma<F32>::V4 &a1) {
    if constexpr (F32) {
        a0 = *reinterpret_cast<const f4 *>(X + R * rowlen + 4 * ((8 * kq + g) ^ (R & 7)));
        a1 = *reinterpret_cast<const f4 *>(X + R * rowlen + 4 * ((8 * kq + 4 + g) ^ (R & 7)));
    } else {
        const h8 v = *reinterpret_cast<const h8 *>(X + R * rowlen + 8 * ((4 * kq + g) ^ img_swz<false>(R, rowlen)));
        a0 = h4{v[0], v[1], v[2], v[3]};
        a1 = h4{v[4], v[5], v[6], v[7]};
    }
}

// Lower-triangular 16x16 tiles (rt >= ct) of a 64x64 matrix, numbered 0..9.
__host__ __device__ constexpr int tri_index(int rt, int ct) { return rt * (rt + 1) / 2 + ct; }

// One step j of the column-oriented forward substitution in a 16-lane row:
// x[r] -= L[r][j] x[j] for r > j, where lane j of the row holds L[r][j] in
// lv[r].  One v_fmac_f32_dpp per update: its first source is taken from lane j
// of the row (DPP row_newbcast:j) and negated by the source modifier.  The
// compiler does not fuse a separate DPP move into the multiply-add, which
// doubled the instruction count.  lv must come straight from LDS loads: a DPP
// source written by a vector instruction needs two wait states that the
// compiler cannot see inside the assembly.
template <int J>
__device__ __forceinline__ void subst_step(const float (&lv)[16], float (&x)[16]) {
#pragma unroll
    for (int r = J + 1; r < 16; ++r)
        asm("v_fmac_f32_dpp %0, -%1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
            : "+v"(x[r])
            : "v"(lv[r]), "v"(x[J]), "i"(J));
}
template <int... J>
__device__ __forceinline__ void subst_steps(const float (&lv)[16], float (&x)[16], std::integer_sequence<int, J...>) {
    (subst_step<J>(lv, x), ...);
}

// Off-diagonal blocks of X = (I + L)^{-1}, 16x16 blocks, diagonal blocks already
// in Xw:  X[i][j] = -X[i][i] sum_{mb=j}^{i-1} L[i][mb] X[mb][j], one column block
// at a time.  A column's finished blocks stay in accumulator layout, the B
// operand of the next product.  Lf holds the A-operand fragments of L's
// off-diagonal blocks; Xw is this wave's block-packed row-major copy of X.
// All ten blocks are also returned in accumulator layout (Xa: lane (m, g) holds
// X[16i + 4g + s][16j + m]).
template <bool F32>
__device__ __forceinline__ void inverse_offdiag(float *Xw, const f4 (&Lf)[10], int m, int g, f4 (&Xa)[10]) {
    typedef mma<F32> M;
#pragma unroll
    for (int s = 0; s < 4; ++s) Xa[tri_index(3, 3)][s] = Xw[tri_index(3, 3) * 256 + (4 * g + s) * 16 + m];
#pragma unroll
    for (int jb = 0; jb < 3; ++jb) {
        f4 Xc[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) Xc[jb][s] = Xw[tri_index(jb, jb) * 256 + (4 * g + s) * 16 + m];
        Xa[tri_index(jb, jb)] = Xc[jb];
#pragma unroll
        for (int ib = jb + 1; ib < 4; ++ib) {
            f4 Tacc = {0, 0, 0, 0};
#pragma unroll
            for (int mb = jb; mb < ib; ++mb)
                Tacc = M::block(Tacc, M::from_f4(Lf[tri_index(ib, mb)]), M::from_f4(Xc[mb]));
            const f4 dv = *reinterpret_cast<const f4 *>(Xw + tri_index(ib, ib) * 256 + m * 16 + 4 * g);
            f4 Xn = {0, 0, 0, 0};
            Xn = -M::block(Xn, M::from_f4(dv), M::from_f4(Tacc));
            Xc[ib] = Xn;
            Xa[tri_index(ib, jb)] = Xn;
#pragma unroll
            for (int s = 0; s < 4; ++s) Xw[tri_index(ib, jb) * 256 + (4 * g + s) * 16 + m] = Xn[s];
        }
    }
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace gdn
