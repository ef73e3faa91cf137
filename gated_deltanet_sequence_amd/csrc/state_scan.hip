// state_scan.hip -- inter-chunk state scan with fused output (method and
// notation in prefill_common.h).
//
// Per chunk, with R' = V - gamma (.) (K S) the residual of the chunk-start
// state S, the chunk-local kernel has prepared two 64 x 64 lower-triangular
// matrices (operand fragments "pairs"):
//   Ae = diag(eta) A diag(beta)   so that   eta (.) Delta = Ae R'
//   Ao = A_qk A diag(beta)        so that   A_qk Delta    = Ao R'
// and the scan runs, all on the matrix cores:
//   P = K S,  R' = V - gamma (.) P
//   O = gamma (.) (Q S) + Ao R'
//   S = gamma_C S + K^T (Ae R')
// The columns of S are independent recurrences, so work-groups split the
// value dimension.  Accumulator tiles of S and R' feed the next product as B
// operands directly (see gdn_device.h), so the state never leaves registers.
//
// Two kernels: scan_split_kernel (float16 operands, bfloat16 inputs) and
// state_scan_kernel (float32 operands, float32 inputs), described at each.
#include <type_traits>

#include "prefill_common.h"

namespace gdn {

typedef __attribute__((address_space(3))) void lds_void_t;

template <bool F32, typename TIn, int DK, int NW, int NL>
struct ScanCfg {
    typedef typename mma<F32>::E E;
    static constexpr int NCOL = 16 * NW;                     // state columns per work-group
    static constexpr size_t IMG_BYTES = (size_t)C * DK * sizeof(E);
    static constexpr int VSPR = NCOL * (int)sizeof(TIn) / 16; // 16-byte slots per V / output row
    static constexpr int VEPS = 16 / (int)sizeof(TIn);       // elements per slot
    static constexpr size_t FRAG_BYTES = (size_t)NPAIR * 64 * 8 * sizeof(E);
    static constexpr size_t TILE_BYTES = (size_t)C * NCOL * sizeof(TIn);  // V or output tile
    static constexpr size_t OFF_Q = 0;
    static constexpr size_t OFF_K = OFF_Q + IMG_BYTES;
    static constexpr size_t OFF_T = OFF_K + IMG_BYTES;
    static constexpr size_t OFF_V = OFF_T + IMG_BYTES;
    static constexpr size_t OFF_TK = OFF_V + TILE_BYTES;
    static constexpr size_t OFF_AF = OFF_TK + (size_t)C * 16;
    static constexpr size_t OFF_QF = OFF_AF + FRAG_BYTES;
    static constexpr size_t BUF = OFF_QF + FRAG_BYTES;
    static constexpr int NBUF = (2 * BUF + 2 * TILE_BYTES <= 160 * 1024) ? 2 : 1;
    static constexpr size_t OFF_O = NBUF * BUF;              // two output tiles follow the buffers
    static constexpr size_t LDS = OFF_O + 2 * TILE_BYTES;
    static constexpr int IMG_UNITS = (int)(IMG_BYTES / 1024);   // 1 KB copies per image
    static constexpr int FRAG_UNITS = (int)(FRAG_BYTES / 1024);
    static constexpr int TILE_UNITS = (int)(TILE_BYTES / 1024);
    static_assert(IMG_BYTES % 1024 == 0 && TILE_BYTES % 1024 == 0 && FRAG_BYTES % 1024 == 0, "copy units");
    static_assert(IMG_UNITS % NL == 0 && FRAG_UNITS % NL == 0 && TILE_UNITS % NL == 0, "copy split");
    static_assert(VSPR >= 4 && (VSPR & (VSPR - 1)) == 0, "V slots");
    static_assert(LDS <= 160 * 1024, "LDS");
    // output stores a loader wave issues per chunk (they stay in flight past its load wait)
    static constexpr int OSTORES = TILE_UNITS / NL;
};

// The 8 operand values of one pair step stored contiguously (fragment layout).
template <bool F32>
__device__ __forceinline__ void ld_pair(const typename mma<F32>::E *p, typename mma<F32>::V4 &a0,
                                        typename mma<F32>::V4 &a1) {
    if constexpr (F32) {
        a0 = *reinterpret_cast<const f4 *>(p);
        a1 = *reinterpret_cast<const f4 *>(p + 4);
    } else {
        const h8 v = *reinterpret_cast<const h8 *>(p);
        a0 = h4{v[0], v[1], v[2], v[3]};
        a1 = h4{v[4], v[5], v[6], v[7]};
    }
}

__device__ __forceinline__ float lds_in(const float *p) { return *p; }
__device__ __forceinline__ float lds_in(const bf16_t *p) {
    return bf16_to_f32(*reinterpret_cast<const uint16_t *>(p));
}
__device__ __forceinline__ void lds_out(float *p, float x) { *p = x; }
__device__ __forceinline__ void lds_out(bf16_t *p, float x) {
    *reinterpret_cast<__bf16 *>(p) = (__bf16)x;
}

// s_waitcnt with vmcnt(n) and no wait on the other counters (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// work-group barrier without a memory fence: each wave completes what the
// others need (its LDS writes, or its loads into LDS) explicitly before it
__device__ __forceinline__ void bare_barrier() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// G2: the channel-wise decay (Gated DeltaNet-2, float32): the images are the
// per-value-head Qt, Et and Kh^T, V is Z, the fragments are A and Aq A, and
// the per-chunk record is e^{G_C} per key channel: R' = Z - Et S,
// O = Qt S + (Aq A) R', S = diag(e^{G_C}) S + Kh^T (A R').
template <bool F32, typename TIn, int DK, int DV, int NW, int NL, bool G2 = false>
__global__ __launch_bounds__(64 * (NW + NL)) void state_scan_kernel(
    int T, int Hk, int Hv, int NC, const TIn *__restrict__ v,
    const float *__restrict__ tok, const typename mma<F32>::E *__restrict__ apair,
    const typename mma<F32>::E *__restrict__ qpair, const typename mma<F32>::E *__restrict__ qimg,
    const typename mma<F32>::E *__restrict__ kimg, const typename mma<F32>::E *__restrict__ timg,
    const float *__restrict__ S0, TIn *__restrict__ out, float *__restrict__ ST) {
    typedef ScanCfg<F32, TIn, DK, NW, NL> CF;
    typedef typename mma<F32>::E E;
    typedef typename mma<F32>::V4 V4;
    static_assert(!G2 || F32, "the channel-wise decay runs here in float32 only");
    constexpr int NCOL = CF::NCOL;
    constexpr int TKB = G2 ? DK * 4 : C * 8;  // per-chunk record bytes
    static_assert(TKB <= C * 16 && TKB % 16 == 0, "record slot");
    constexpr int NKB = DK / 16;
    constexpr int NCG = DV / NCOL;

    __shared__ __attribute__((aligned(1024))) char smem[CF::LDS];

    // XCD-aware numbering: work-groups are dealt round-robin to the 8 XCDs, so
    // give each XCD a contiguous range of logical ids (same key head nearby).
    const int nblk = gridDim.x;
    int lid = blockIdx.x;
    if ((nblk & 7) == 0) lid = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
    const int cg = lid % NCG;
    const int hv = (lid / NCG) % Hv;
    const int bb = lid / (NCG * Hv);
    const int hk = hv / (Hv / Hk);
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in a scalar register
    const bool loader = w >= NW;

    if (loader) {
        // ================= loader waves =================
        const int l = w - NW;
        const size_t seq_elems = (size_t)T * Hv * DV;
        auto rsrc = [](const void *p, size_t bytes) {
            return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
        };
        // sequence-bounded V and output; unit-bounded workspace regions
        const __amdgpu_buffer_rsrc_t vres = rsrc(v + (size_t)bb * seq_elems, seq_elems * sizeof(TIn));
        const __amdgpu_buffer_rsrc_t ores = rsrc(out + (size_t)bb * seq_elems, seq_elems * sizeof(TIn));
        const size_t ku0 = ((size_t)bb * Hk + hk) * NC, vu0 = ((size_t)bb * Hv + hv) * NC;
        const size_t iu0 = G2 ? vu0 : ku0;  // images per value head (channel-wise decay) or per key head
        const __amdgpu_buffer_rsrc_t rq = rsrc(qimg + iu0 * C * DK, (size_t)NC * CF::IMG_BYTES);
        const __amdgpu_buffer_rsrc_t rk = rsrc(kimg + iu0 * C * DK, (size_t)NC * CF::IMG_BYTES);
        const __amdgpu_buffer_rsrc_t rt = rsrc(timg + iu0 * C * DK, (size_t)NC * CF::IMG_BYTES);
        const __amdgpu_buffer_rsrc_t ra = rsrc(apair + vu0 * (NPAIR * 64 * 8), (size_t)NC * CF::FRAG_BYTES);
        const __amdgpu_buffer_rsrc_t rf = rsrc(qpair + vu0 * (NPAIR * 64 * 8), (size_t)NC * CF::FRAG_BYTES);
        const __amdgpu_buffer_rsrc_t rtk = rsrc(tok + vu0 * (TKB / 4), (size_t)NC * TKB);
        const int lane16 = lane * 16;
        // 16-byte slot of this lane in tile unit u: row, swizzled piece, element offset
        auto tile_slot = [&](int u, int &row, int &piece) {
            const int slot = u * 64 + lane;
            row = slot / CF::VSPR;
            piece = (slot % CF::VSPR) ^ ((row >> 2) & (CF::VSPR - 1));
        };

        // copy chunk n into LDS buffer `buf` (1 KB per instruction, direct to LDS)
        auto stage = [&](int n, int buf) {
            char *base = smem + (size_t)buf * CF::BUF;
            const int io = n * (int)CF::IMG_BYTES, fo = n * (int)CF::FRAG_BYTES;
#pragma unroll
            for (int i = 0; i < CF::IMG_UNITS / NL; ++i) {
                const int u = (l + NL * i) * 1024;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void_t *)(base + CF::OFF_Q + u), 16, lane16, io + u, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t *)(base + CF::OFF_K + u), 16, lane16, io + u, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, (lds_void_t *)(base + CF::OFF_T + u), 16, lane16, io + u, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < CF::FRAG_UNITS / NL; ++i) {
                const int u = (l + NL * i) * 1024;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t *)(base + CF::OFF_AF + u), 16, lane16, fo + u, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rf, (lds_void_t *)(base + CF::OFF_QF + u), 16, lane16, fo + u, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < CF::TILE_UNITS / NL; ++i) {
                const int u = l + NL * i;
                int row, piece;
                tile_slot(u, row, piece);
                const int voff = ((n * C + row) * Hv + hv) * DV + NCOL * cg + piece * CF::VEPS;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vres, (lds_void_t *)(base + CF::OFF_V + u * 1024), 16,
                                                         voff * (int)sizeof(TIn), 0, 0, 0);
            }
            if (l == 0 && lane < TKB / 16)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rtk, (lds_void_t *)(base + CF::OFF_TK), 16, lane16, n * TKB, 0, 0);
        };
        // write chunk n's output rows from LDS output tile (n & 1), 16 bytes per lane
        auto store_rows = [&](int n) {
            const char *ob = smem + CF::OFF_O + (size_t)(n & 1) * CF::TILE_BYTES;
#pragma unroll
            for (int i = 0; i < CF::TILE_UNITS / NL; ++i) {
                const int u = l + NL * i;
                int row, piece;
                tile_slot(u, row, piece);
                typedef uint32_t u4v __attribute__((ext_vector_type(4)));
                const u4v val = *reinterpret_cast<const u4v *>(ob + u * 1024 + lane16);
                const int ooff = ((n * C + row) * Hv + hv) * DV + NCOL * cg + piece * CF::VEPS;
                __builtin_amdgcn_raw_buffer_store_b128(val, ores, ooff * (int)sizeof(TIn), 0, 0);
            }
        };

        stage(0, 0);
        wait_vmcnt<0>();
        bare_barrier();
        for (int n = 0; n < NC; ++n) {
            const bool more = n + 1 < NC;
            if (CF::NBUF == 2) {
                if (more) stage(n + 1, (n + 1) & 1);
                if (n > 0) {
                    store_rows(n - 1);
                    wait_vmcnt<CF::OSTORES>();  // loads landed; this chunk's stores may still fly
                } else {
                    wait_vmcnt<0>();
                }
                bare_barrier();
            } else {
                bare_barrier();                 // compute waves are done with the single buffer
                if (more) stage(n + 1, 0);
                store_rows(n);
                wait_vmcnt<CF::OSTORES>();
                bare_barrier();
            }
        }
        if (CF::NBUF == 2 && NC > 0) store_rows(NC - 1);
        return;
    }

    // ================= compute waves =================
    const int lc = 16 * w + m;              // column within the group
    const int col = NCOL * cg + lc;         // state column

    // state S[16kb + 4g + i][col] in accumulator tiles
    f4 S[NKB];
    const size_t sb = ((size_t)bb * Hv + hv) * DK * DV;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[kb][i] = S0 ? S0[sb + (size_t)(16 * kb + 4 * g + i) * DV + col] : 0.f;

    // element (row, lc) of a V / output tile (16-byte slots swizzled like the loaders')
    auto tile_index = [&](int row) {
        const int piece = lc / CF::VEPS;
        return row * NCOL + ((piece ^ ((row >> 2) & (CF::VSPR - 1))) * CF::VEPS) + lc % CF::VEPS;
    };

    bare_barrier();  // chunk 0 staged
    for (int n = 0; n < NC; ++n) {
        const char *base = smem + (size_t)(n % CF::NBUF) * CF::BUF;
        const E *Qs = reinterpret_cast<const E *>(base + CF::OFF_Q);
        const E *Ks = reinterpret_cast<const E *>(base + CF::OFF_K);
        const E *Kt = reinterpret_cast<const E *>(base + CF::OFF_T);
        const TIn *Vs = reinterpret_cast<const TIn *>(base + CF::OFF_V);
        const float *Tq = reinterpret_cast<const float *>(base + CF::OFF_TK);  // [gamma | gamma by lane][64]
        const E *Af = reinterpret_cast<const E *>(base + CF::OFF_AF) + lane * 8;
        const E *Qf = reinterpret_cast<const E *>(base + CF::OFF_QF) + lane * 8;
        TIn *Os = reinterpret_cast<TIn *>(smem + CF::OFF_O + (size_t)(n & 1) * CF::TILE_BYTES);
        // token quantity X of this lane's rows 16r + 4g + i, i = 0..3
        auto tokq = [&](int x, int r) { return *reinterpret_cast<const f4 *>(Tq + 64 * x + 16 * r + 4 * g); };

        // operands of the residual, read ahead of the products that need them
        f4 ga[4], vv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            ga[r] = G2 ? f4{1, 1, 1, 1} : tokq(0, r);
#pragma unroll
            for (int i = 0; i < 4; ++i) vv[r][i] = lds_in(Vs + tile_index(16 * r + 4 * g + i));
        }

        V4 Sb[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) Sb[kb] = mma<F32>::from_f4(S[kb]);

        // ---- P = K S, Qa = Q S: contraction step outer, 8 independent accumulators;
        //      the operands of step kq+1 are read while step kq's products run
        f4 P[4], Qa[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) P[r] = Qa[r] = f4{0, 0, 0, 0};
        V4 kf[2][4][2], qf[2][4][2];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            img_pair<F32>(Ks, DK, 16 * r + m, 0, g, kf[0][r][0], kf[0][r][1]);
            img_pair<F32>(Qs, DK, 16 * r + m, 0, g, qf[0][r][0], qf[0][r][1]);
        }
#pragma unroll
        for (int kq = 0; kq < DK / 32; ++kq) {
            const int cb = kq & 1;
            if (kq + 1 < DK / 32) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    img_pair<F32>(Ks, DK, 16 * r + m, kq + 1, g, kf[cb ^ 1][r][0], kf[cb ^ 1][r][1]);
                    img_pair<F32>(Qs, DK, 16 * r + m, kq + 1, g, qf[cb ^ 1][r][0], qf[cb ^ 1][r][1]);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                P[r] = mma<F32>::pair(P[r], kf[cb][r][0], kf[cb][r][1], Sb[2 * kq], Sb[2 * kq + 1]);
                Qa[r] = mma<F32>::pair(Qa[r], qf[cb][r][0], qf[cb][r][1], Sb[2 * kq], Sb[2 * kq + 1]);
            }
        }

        // operands of Delta and O, read while the products above drain
        V4 afr[NPAIR][2], qfr[NPAIR][2];
#pragma unroll
        for (int p = 0; p < NPAIR; ++p) {
            ld_pair<F32>(Af + p * 512, afr[p][0], afr[p][1]);
            ld_pair<F32>(Qf + p * 512, qfr[p][0], qfr[p][1]);
        }

        // ---- R' = V - gamma P  (channel-wise decay: Z - Et S, the decay is in the image)
        V4 Rb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) Rb[r] = mma<F32>::from_f4(G2 ? vv[r] - P[r] : vv[r] - ga[r] * P[r]);

        // ---- eta Delta = Ae R'
        V4 De[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            f4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int qq = 0; qq <= r / 2; ++qq) {
                const int p = pair_index(r, qq);
                acc = mma<F32>::pair(acc, afr[p][0], afr[p][1], Rb[2 * qq], Rb[2 * qq + 1]);
            }
            De[r] = mma<F32>::from_f4(acc);
        }

        // K^T operands of the state update, read ahead of it
        V4 tf[NKB][2][2];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) img_pair<F32>(Kt, C, 16 * kb + m, qq, g, tf[kb][qq][0], tf[kb][qq][1]);

        // ---- O = gamma Qa + Ao R', into the LDS output tile (the read-out
        //      scale is already folded into Q and Ao)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            f4 acc = G2 ? Qa[r] : ga[r] * Qa[r];
#pragma unroll
            for (int qq = 0; qq <= r / 2; ++qq) {
                const int p = pair_index(r, qq);
                acc = mma<F32>::pair(acc, qfr[p][0], qfr[p][1], Rb[2 * qq], Rb[2 * qq + 1]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) lds_out(Os + tile_index(16 * r + 4 * g + i), acc[i]);
        }

        // ---- S = gamma_C S + K^T (eta Delta)  (channel-wise: e^{G_C} of row 16 kb + 4 g + i)
        const float gC = Tq[C - 1];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            f4 acc = G2 ? *reinterpret_cast<const f4 *>(Tq + 16 * kb + 4 * g) * S[kb] : gC * S[kb];
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) acc = mma<F32>::pair(acc, tf[kb][qq][0], tf[kb][qq][1], De[2 * qq], De[2 * qq + 1]);
            S[kb] = acc;
        }

        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the output tile is written
        bare_barrier();
        if (CF::NBUF == 1) bare_barrier();   // the loaders refill the single buffer
    }

    if (ST) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) ST[sb + (size_t)(16 * kb + 4 * g + i) * DV + col] = S[kb][i];
    }
}

// ---------------------------------------------------------------------------
// Role-split scan (float16 operands, bfloat16 inputs and outputs).
//
// One work-group per (sequence, value head, 32 state columns), six waves with
// distinct roles.  Waves w and w + 4 share a SIMD; the two state waves get a
// SIMD each, every other SIMD holds an output wave and a loader wave.
//   two state waves (waves 2 and 3), one per 16-column tile: each holds its
//     S[d_k][16] in accumulator tiles and runs the recurrence P = K S,
//     R' = V - gamma P, S = gamma_C S + K^T (Ae R'); the two tiles are
//     independent, so the chunk-to-chunk chain of each wave carries half the
//     vector and matrix work of one 32-column wave (the K and K^T operand
//     reads are not halved: both waves read them).  Per chunk each hands the
//     float16 operand pairs of its chunk-start S and of R' to the output waves
//     through LDS;
//   two output waves (waves 0 and 1), one chunk behind, each for two of the
//     four 16-token row tiles and both column tiles:
//     O^T = gamma (S^T Q^T) + R'^T Ao^T.  The transposed products take the very
//     same operand registers, and their accumulators give each lane 4
//     consecutive output columns of one token, written with one 8-byte store;
//   two loader waves: copy inputs into LDS with direct-to-LDS buffer loads --
//     wave 5 K, V, Ae and gamma for the state waves, wave 4 Q, Ao and gamma
//     for the output waves; the images two chunks ahead, the rest one ahead.
// Only the state waves are on the chunk-to-chunk critical path.  One barrier
// per chunk.
// ---------------------------------------------------------------------------
typedef short s4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4 lds_s4;

// Operand pair of image row R as one 8-value register group (float16 images).
__device__ __forceinline__ h8 img_h8(const _Float16 *X, int rowlen, int R, int kq, int g) {
    return *reinterpret_cast<const h8 *>(X + R * rowlen + 8 * ((4 * kq + g) ^ img_swz<false>(R, rowlen)));
}

template <typename TIn, int DK, int NL, bool G2, int NT_ = 2>
struct SplitCfg {
    static constexpr int NT = NT_;                                 // 16-column tiles (state waves) per work-group
    static constexpr int NCOL = 16 * NT;
    static constexpr int NKQ = DK / 32;                            // 32-deep contraction steps over d_k
    static constexpr int IMG_BYTES = C * DK * 2;
    static constexpr int FRAG_BYTES = NPAIR * 64 * 8 * 2;
    // per-chunk record of the state waves: gamma twice (two token orders), or
    // for the channel-wise decay e^{G_C} per key channel; the output waves'
    // gamma record (none for the channel-wise decay, folded into its Q image)
    static constexpr int STK_BYTES = G2 ? DK * 4 : C * 8, OTK_BYTES = G2 ? 0 : C * 8;
    static constexpr int TILE_BYTES = C * NCOL * 2;                // V (or write-logit) tile, bfloat16
    static constexpr int VSPR = NCOL * 2 / 16;                     // 16-byte slots per V row
    static constexpr int VEPS = 8;                                 // elements per slot
    // State-wave inputs: the image for P = K S (K; Et for the channel-wise
    // decay), the image of the state update's K^T operands (the same K image;
    // a separate Kh image for the channel-wise decay), V (and for the
    // channel-wise decay the write-gate logits: z = sigmoid(write) v is formed
    // by the state waves), Ae, the record.
    // Output-wave inputs: the Q image, Ao, gamma.  Every stream has NSB (NOB)
    // LDS buffers, issued NSB-1 (NOB-1) chunks ahead: 3 for the scalar decay,
    // 2 for the channel-wise decay (its two state images fill LDS).  The
    // hand-over is single-buffered (two barriers per chunk).
    static constexpr int S_K = 0, S_KH = G2 ? S_K + IMG_BYTES : S_K, S_V = S_KH + IMG_BYTES,
                         S_W = S_V + TILE_BYTES, S_A = S_W + (G2 ? TILE_BYTES : 0), S_TK = S_A + FRAG_BYTES,
                         S_BUF = S_TK + STK_BYTES;
    static constexpr int O_Q = 0, O_F = O_Q + IMG_BYTES, O_TK = O_F + FRAG_BYTES, O_BUF = O_TK + OTK_BYTES;
    // hand-over: S (d_k x 16) and R' (64 x 16) of each column tile as operand pairs, 1 KB each
    static constexpr int X_S = 0, X_R = NT * NKQ * 1024, X_BUF = X_R + NT * 2 * 1024;
    // buffer depths: three each where they fit in LDS (two chunks of lead), else
    // the state stream keeps three if it can; the channel-wise decay two each
    static constexpr int NSB = G2 ? 2 : (3 * S_BUF + 2 * O_BUF + X_BUF <= 160 * 1024) ? 3 : 2;
    static constexpr int NOB = G2 ? 2 : (NSB * S_BUF + 3 * O_BUF + X_BUF <= 160 * 1024) ? 3 : 2;
    static constexpr int OFF_S = 0, OFF_O = OFF_S + NSB * S_BUF, OFF_X = OFF_O + NOB * O_BUF, LDS = OFF_X + X_BUF;
    static constexpr int IMG_UNITS = IMG_BYTES / 1024, FRAG_UNITS = FRAG_BYTES / 1024,
                         TILE_UNITS = TILE_BYTES / 1024;
    // loads per chunk of the state loader and of the output loader
    static constexpr int STATE_LOADS = (IMG_UNITS + TILE_UNITS) * (G2 ? 2 : 1) + FRAG_UNITS + 1,
                         OUT_LOADS = IMG_UNITS + FRAG_UNITS + (G2 ? 0 : 1);
    static_assert((NSB - 1) * STATE_LOADS < 64 && (NOB - 1) * OUT_LOADS < 64, "vmcnt");
    static_assert(VSPR >= 4 && (VSPR & (VSPR - 1)) == 0, "V slots");
    static_assert(S_BUF % 16 == 0 && O_BUF % 16 == 0, "alignment");
    static_assert(LDS <= 160 * 1024, "LDS");
};

// Loader-wave copies of one chunk's inputs into LDS: 16 bytes per lane per
// instruction, straight from memory into LDS (no registers).  One loader wave
// stages the state-wave inputs, the other the output-wave inputs: each wave's
// loads complete in issue order, so the two streams do not wait on each other.
template <typename TIn, int DK, int NL, bool G2, int NT>
struct SplitLoader {
    typedef SplitCfg<TIn, DK, NL, G2, NT> CF;
    __amdgpu_buffer_rsrc_t vres, wres, rq, rk, rkh, ra, rf, rtk, rgc;
    int lane;
    unsigned vcol;  // element offset of this group's first V column in a token row
    unsigned vrow;  // elements per token row of V (Hv * d_v)

    __device__ __forceinline__ void copy(__amdgpu_buffer_rsrc_t r, char *dst, int src_off) const {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)dst, 16, lane * 16, src_off, 0, 0);
    }
    // state-wave inputs of chunk n: image(s), V columns, Ae fragments, record (STATE_LOADS loads)
    __device__ __forceinline__ void stage_state(char *smem, int n, int buf) const {
        char *base = smem + CF::OFF_S + buf * CF::S_BUF;
        const int io = n * CF::IMG_BYTES, fo = n * CF::FRAG_BYTES;
#pragma unroll
        for (int u = 0; u < CF::IMG_UNITS; ++u) copy(rk, base + CF::S_K + u * 1024, io + u * 1024);
        if constexpr (G2) {
#pragma unroll
            for (int u = 0; u < CF::IMG_UNITS; ++u) copy(rkh, base + CF::S_KH + u * 1024, io + u * 1024);
        }
#pragma unroll
        for (int u = 0; u < CF::TILE_UNITS; ++u) {
            const int slot = u * 64 + lane;
            const int row = slot / CF::VSPR;
            const int piece = (slot % CF::VSPR) ^ ((row >> 2) & (CF::VSPR - 1));
            const unsigned voff = ((unsigned)(n * C + row) * vrow + vcol + piece * CF::VEPS) * (unsigned)sizeof(TIn);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vres, (lds_void_t *)(base + CF::S_V + u * 1024), 16, (int)voff, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < CF::FRAG_UNITS; ++u) copy(ra, base + CF::S_A + u * 1024, fo + u * 1024);
        if (lane < CF::STK_BYTES / 16) copy(G2 ? rgc : rtk, base + CF::S_TK, n * CF::STK_BYTES);
    }
    // the channel-wise decay's state-wave inputs in two portions by the time
    // the state waves read them: "early" (the Et image, V and the write
    // logits, A; read one chunk ahead, during the previous chunk's state
    // update) and "late" (the Kh image and e^{G_C}; read during the chunk's own
    // phases A and B)
    static constexpr int EARLY_LOADS = CF::IMG_UNITS + 2 * CF::TILE_UNITS + CF::FRAG_UNITS,
                         LATE_LOADS = CF::IMG_UNITS + 1;
    __device__ __forceinline__ void stage_early(char *smem, int n, int buf) const {
        char *base = smem + CF::OFF_S + buf * CF::S_BUF;
        const int io = n * CF::IMG_BYTES, fo = n * CF::FRAG_BYTES;
#pragma unroll
        for (int u = 0; u < CF::IMG_UNITS; ++u) copy(rk, base + CF::S_K + u * 1024, io + u * 1024);
#pragma unroll
        for (int u = 0; u < CF::TILE_UNITS; ++u) {
            const int slot = u * 64 + lane;
            const int row = slot / CF::VSPR;
            const int piece = (slot % CF::VSPR) ^ ((row >> 2) & (CF::VSPR - 1));
            const unsigned voff = ((unsigned)(n * C + row) * vrow + vcol + piece * CF::VEPS) * (unsigned)sizeof(TIn);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vres, (lds_void_t *)(base + CF::S_V + u * 1024), 16, (int)voff, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, (lds_void_t *)(base + CF::S_W + u * 1024), 16, (int)voff, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < CF::FRAG_UNITS; ++u) copy(ra, base + CF::S_A + u * 1024, fo + u * 1024);
    }
    __device__ __forceinline__ void stage_late(char *smem, int n, int buf) const {
        char *base = smem + CF::OFF_S + buf * CF::S_BUF;
        const int io = n * CF::IMG_BYTES;
#pragma unroll
        for (int u = 0; u < CF::IMG_UNITS; ++u) copy(rkh, base + CF::S_KH + u * 1024, io + u * 1024);
        if (lane < CF::STK_BYTES / 16) copy(rgc, base + CF::S_TK, n * CF::STK_BYTES);
    }
    // output-wave inputs of chunk n: Q image, Ao fragments, gamma (OUT_LOADS loads)
    __device__ __forceinline__ void stage_out(char *smem, int n, int buf) const {
        char *base = smem + CF::OFF_O + buf * CF::O_BUF;
        const int io = n * CF::IMG_BYTES, fo = n * CF::FRAG_BYTES;
#pragma unroll
        for (int u = 0; u < CF::IMG_UNITS; ++u) copy(rq, base + CF::O_Q + u * 1024, io + u * 1024);
#pragma unroll
        for (int u = 0; u < CF::FRAG_UNITS; ++u) copy(rf, base + CF::O_F + u * 1024, fo + u * 1024);
        if constexpr (!G2)
            if (lane < CF::OTK_BYTES / 16) copy(rtk, base + CF::O_TK, n * CF::OTK_BYTES);
    }
};

template <typename TIn, int DK, int DV, int NL, bool G2, int NT_>
__global__ __launch_bounds__(64 * (NT_ + 2 + NL)) void scan_split_kernel(
    int T, int Hk, int Hv, int NC, const void *__restrict__ v, const void *__restrict__ wlog,
    const float *__restrict__ tok, const _Float16 *__restrict__ apair, const _Float16 *__restrict__ qpair,
    const _Float16 *__restrict__ qimg, const _Float16 *__restrict__ kimg,
    const _Float16 *__restrict__ khimg, const float *__restrict__ gcrec,
    const float *__restrict__ S0, TIn *__restrict__ out, float *__restrict__ ST) {
    static_assert(sizeof(TIn) == 2, "bfloat16 inputs");
    static_assert(NL == 2, "two loader waves");
    static_assert(NT_ == 2 || (NT_ == 4 && !G2), "2 or 4 column tiles (4: scalar decay)");
    typedef SplitCfg<TIn, DK, NL, G2, NT_> CF;
    typedef _Float16 E;
    constexpr int NT = CF::NT, NCOL = CF::NCOL, NKB = DK / 16, NKQ = CF::NKQ, NCG = DV / NCOL;
    // Wave roles.  Waves w and w + 4 share a SIMD.  Two column tiles: output
    // waves 0, 1, state waves 2, 3, loaders 4, 5 (each state wave alone on its
    // SIMD).  Four column tiles: state waves 0..3 (one per SIMD), output
    // waves 4, 5 and loaders 6, 7 beside them.
    constexpr int W_STATE = NT == 2 ? 2 : 0, W_OUT = NT == 2 ? 0 : 4, W_LOAD = NT == 2 ? 4 : 6;

    __shared__ __attribute__((aligned(1024))) char smem[CF::LDS];

    // XCD-aware numbering: work-groups are dealt round-robin to the 8 XCDs, so
    // give each XCD a contiguous range of logical ids (same key head nearby).
    const int nblk = gridDim.x;
    int lid = blockIdx.x;
    if ((nblk & 7) == 0) lid = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
    const int cg = lid % NCG;
    const int hv = (lid / NCG) % Hv;
    const int bb = lid / (NCG * Hv);
    const int hk = hv / (Hv / Hk);
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t seq_elems = (size_t)T * Hv * DV;
    auto rsrc = [](const void *p, size_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
    };

    if (w >= W_LOAD) {
        // ================= loader waves =================
        const size_t ku0 = ((size_t)bb * Hk + hk) * NC, vu0 = ((size_t)bb * Hv + hv) * NC;
        const size_t iu0 = G2 ? vu0 : ku0;  // images per value head (channel-wise decay) or per key head
        SplitLoader<TIn, DK, NL, G2, NT> ld;
        ld.vres = rsrc((const char *)v + (size_t)bb * seq_elems * 2, seq_elems * 2);
        if constexpr (G2) ld.wres = rsrc((const char *)wlog + (size_t)bb * seq_elems * 2, seq_elems * 2);
        ld.rq = rsrc(qimg + iu0 * C * DK, (size_t)NC * CF::IMG_BYTES);
        ld.rk = rsrc(kimg + iu0 * C * DK, (size_t)NC * CF::IMG_BYTES);
        if constexpr (G2) ld.rkh = rsrc(khimg + iu0 * C * DK, (size_t)NC * CF::IMG_BYTES);
        ld.ra = rsrc(apair + vu0 * (NPAIR * 64 * 8), (size_t)NC * CF::FRAG_BYTES);
        ld.rf = rsrc(qpair + vu0 * (NPAIR * 64 * 8), (size_t)NC * CF::FRAG_BYTES);
        if constexpr (G2) ld.rgc = rsrc(gcrec + vu0 * DK, (size_t)NC * CF::STK_BYTES);
        else ld.rtk = rsrc(tok + vu0 * C * 2, (size_t)NC * CF::STK_BYTES);
        ld.lane = lane;
        ld.vcol = (unsigned)(hv * DV + NCOL * cg);
        ld.vrow = (unsigned)(Hv * DV);

        // Barriers, the same sequence in every wave: P(-1), then per chunk n
        // P(n) -- chunk n+1's state-wave inputs, chunk n's output-wave inputs
        // and chunk n's hand-over are in LDS -- and F(n) -- the output waves
        // have read chunk n's hand-over.  After P(n) the state waves are done
        // with chunk n's inputs and the output waves with chunk n-1's: chunk
        // n+3's state inputs and chunk n+2's output inputs are issued into
        // those buffers right then, and waited for just before the barrier
        // that publishes them, more than two chunk intervals later.  Loads
        // complete in issue order, so waiting until only the newest chunk's
        // loads are outstanding suffices.
        // wait until at most k chunks' loads of this stream are in flight
        // (at most K chunks ahead: K = buffers - 1 <= 2)
        auto wait_chunks = [](int k, auto LOADS, auto KMAX) {
            constexpr int L = decltype(LOADS)::value, K = decltype(KMAX)::value;
            if (k <= 0) wait_vmcnt<0>();
            else if (K < 2 || k == 1) wait_vmcnt<L>();
            else wait_vmcnt<(K < 2 ? 0 : 2 * L)>();
        };
        if (G2 && w == W_LOAD + 1) {
            // Channel-wise decay, two state buffers: chunk m lives in buffer
            // m % 2.  Its early portion is read during E(m-1) (from P(m-1) to
            // F(m-1)), its late portion during A(m) and B(m) (from F(m-1) to
            // P(m)).  So the early portion of chunk n+3 is issued after F(n),
            // the late portion of chunk n+2 after P(n), each more than one
            // chunk interval before it is needed.  Waits count loads issued
            // after the awaited ones (in-order completion).
            constexpr int EL = decltype(ld)::EARLY_LOADS, LL = decltype(ld)::LATE_LOADS;
            auto wait_for = [](bool a_early, bool a_late) {  // loads issued after the awaited ones
                if (a_early && a_late) wait_vmcnt<EL + LL>();
                else if (a_early) wait_vmcnt<EL>();
                else if (a_late) wait_vmcnt<LL>();
                else wait_vmcnt<0>();
            };
            // at most 63 loads in flight (the width of the wave's counter):
            // before issuing L more, wait until at most 63 - L are outstanding
            auto early = [&](int m, int buf) { wait_vmcnt<63 - EL>(); ld.stage_early(smem, m, buf); };
            auto late = [&](int m, int buf) { wait_vmcnt<63 - LL>(); ld.stage_late(smem, m, buf); };
            if (NC > 0) {
                early(0, 0);
                late(0, 0);
            }
            if (NC > 1) {
                early(1, 1);
                late(1, 1);
            }
            wait_for(NC > 1, NC > 1);
            bare_barrier();  // P(-1): chunk 0
            wait_for(false, NC > 1);
            bare_barrier();  // P(0): early portion of chunk 1
            if (NC > 2) early(2, 0);  // chunk 0's early portion was read before P(0)
            for (int n = 0; n < NC; ++n) {
                if (n + 2 < NC) late(n + 2, n & 1);
                if (n + 1 < NC) wait_for(n + 2 < NC, n + 2 < NC);  // late portion of chunk n+1
                bare_barrier();  // F(n)
                if (n + 3 < NC) early(n + 3, (n + 1) & 1);
                if (n + 1 < NC) {
                    wait_for(n + 3 < NC, n + 2 < NC);  // early portion of chunk n+2
                    bare_barrier();  // P(n+1)
                }
            }
        } else if (w == W_LOAD + 1) {
            // state-wave inputs: chunk m is read from P(m-1) to P(m), buffer
            // m % NSB; chunk n+NSB is issued after P(n)
            const std::integral_constant<int, CF::STATE_LOADS> SL;
            const std::integral_constant<int, CF::NSB - 1> SK;
            const int npre = NC < CF::NSB ? NC : CF::NSB;
            for (int j = 0; j < npre; ++j) ld.stage_state(smem, j, j);
            wait_chunks(npre - 1, SL, SK);
            bare_barrier();  // P(-1): chunk 0
            wait_chunks(npre - 2, SL, SK);
            bare_barrier();  // P(0): chunk 1
            int sb = 0;      // buffer of chunk n (and of chunk n + NSB)
            for (int n = 0; n < NC; ++n) {
                if (n + CF::NSB < NC) ld.stage_state(smem, n + CF::NSB, sb);
                bare_barrier();  // F(n)
                if (n + 1 < NC) {
                    const int last = n + CF::NSB < NC - 1 ? n + CF::NSB : NC - 1;  // newest chunk issued
                    wait_chunks(last - n - 2, SL, SK);
                    bare_barrier();  // P(n+1): chunk n+2
                }
                sb = sb == CF::NSB - 1 ? 0 : sb + 1;
            }
        } else {
            // output-wave inputs: chunk m is read from P(m) to P(m+1), buffer
            // m % NOB; chunk n+NOB-1 is issued after P(n)
            const std::integral_constant<int, CF::OUT_LOADS> OL;
            const std::integral_constant<int, CF::NOB - 1> OK;
            const int npre = NC < CF::NOB - 1 ? NC : CF::NOB - 1;
            for (int j = 0; j < npre; ++j) ld.stage_out(smem, j, j);
            bare_barrier();  // P(-1)
            wait_chunks(npre - 1, OL, OK);
            bare_barrier();  // P(0): chunk 0
            int ob = CF::NOB - 1;  // buffer of chunk n + NOB - 1
            for (int n = 0; n < NC; ++n) {
                if (n + CF::NOB - 1 < NC) ld.stage_out(smem, n + CF::NOB - 1, ob);
                bare_barrier();  // F(n)
                if (n + 1 < NC) {
                    const int last = n + CF::NOB - 1 < NC - 1 ? n + CF::NOB - 1 : NC - 1;
                    wait_chunks(last - n - 1, OL, OK);
                    bare_barrier();  // P(n+1): chunk n+1
                }
                ob = ob == CF::NOB - 1 ? 0 : ob + 1;
            }
        }
        return;
    }

    if (w >= W_OUT && w < W_OUT + 2) {
        // ================= output waves (one chunk behind) =================
        // wave 0: token row tiles 0 and 3, wave 1: row tiles 1 and 2 (the same
        // number of products each), both column tiles
        const __amdgpu_buffer_rsrc_t ores = rsrc(out + (size_t)bb * seq_elems, seq_elems * sizeof(TIn));
        const unsigned col = NCOL * cg + 4 * g;
        // chunk n from output buffer obi; the hand-over is read first, then
        // F(n) releases it to the state waves
        auto emit = [&](int n, int obi, auto RA, auto RB) {
            const char *ob = smem + CF::OFF_O + obi * CF::O_BUF;
            const E *Qs = reinterpret_cast<const E *>(ob + CF::O_Q);
            const E *Of = reinterpret_cast<const E *>(ob + CF::O_F) + lane * 8;
            const float *Tq = reinterpret_cast<const float *>(ob + CF::O_TK);
            const char *xb = smem + CF::OFF_X;
            h8 Sp[NT][NKQ], Rp[NT][2];
#pragma unroll
            for (int c = 0; c < NT; ++c) {
#pragma unroll
                for (int j = 0; j < NKQ; ++j)
                    Sp[c][j] = *reinterpret_cast<const h8 *>(xb + CF::X_S + (c * NKQ + j) * 1024 + lane * 16);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    Rp[c][j] = *reinterpret_cast<const h8 *>(xb + CF::X_R + (c * 2 + j) * 1024 + lane * 16);
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the hand-over is in registers
            bare_barrier();                      // F(n)
            f4 gam = {1.f, 1.f, 1.f, 1.f};  // the channel-wise decay has it folded into Q
            if constexpr (!G2) gam = *reinterpret_cast<const f4 *>(Tq + 64 + 4 * m);  // tokens m, 16+m, 32+m, 48+m
            auto rows = [&](auto RR) {
                constexpr int r = decltype(RR)::value;
                f4 sq[NT];
#pragma unroll
                for (int c = 0; c < NT; ++c) sq[c] = f4{0, 0, 0, 0};
#pragma unroll
                for (int kq = 0; kq < NKQ; ++kq) {
                    const h8 qf = img_h8(Qs, DK, 16 * r + m, kq, g);
#pragma unroll
                    for (int c = 0; c < NT; ++c) sq[c] = mfma_f16_k32(Sp[c][kq], qf, sq[c]);
                }
                f4 acc[NT];
#pragma unroll
                for (int c = 0; c < NT; ++c) acc[c] = G2 ? sq[c] : gam[r] * sq[c];
#pragma unroll
                for (int qq = 0; qq <= r / 2; ++qq) {
                    const h8 f = *reinterpret_cast<const h8 *>(Of + pair_index(r, qq) * 512);
#pragma unroll
                    for (int c = 0; c < NT; ++c) acc[c] = mfma_f16_k32(Rp[c][qq], f, acc[c]);
                }
                // lane holds O[token 16r + m][col + 16c .. + 3].  With two column
                // tiles a work-group writes half of each 128-byte line (another
                // work-group, often on another XCD, writes the rest): those stores
                // go out non-temporal, which took 3 us off the prefill step by
                // leaving less dirty data in L2 at the kernel's end.  With four
                // tiles the work-group writes whole lines, which L2 merges from
                // four stores: non-temporal there cost 10 % of the scan.
                constexpr int OUT_CPOL = NT == 2 ? 2 : 0;  // 2: nt
                typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
                typedef uint32_t u2v __attribute__((ext_vector_type(2)));
                const unsigned t = (unsigned)(n * C + 16 * r + m);
#pragma unroll
                for (int c = 0; c < NT; ++c) {
                    const bf4 hb = __builtin_convertvector(acc[c], bf4);
                    u2v bits;
                    __builtin_memcpy(&bits, &hb, 8);
                    __builtin_amdgcn_raw_buffer_store_b64(bits, ores, (int)(((t * Hv + hv) * DV + col + 16 * c) * 2u), 0, OUT_CPOL);
                }
            };
            rows(RA);
            rows(RB);
        };
        bare_barrier();  // P(-1)
        int ob = 0;      // buffer of chunk n
        for (int n = 0; n < NC; ++n) {
            bare_barrier();  // P(n)
            if (w == W_OUT) emit(n, ob, std::integral_constant<int, 0>(), std::integral_constant<int, 3>());
            else emit(n, ob, std::integral_constant<int, 1>(), std::integral_constant<int, 2>());
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this chunk's LDS reads are done
            ob = ob == CF::NOB - 1 ? 0 : ob + 1;
        }
        return;
    }

    // ================= state waves: column tile c = w - W_STATE =================
    const int c = w - W_STATE;
    f4 S[NKB];
    const size_t sb = ((size_t)bb * Hv + hv) * DK * DV;
    const int scol = NCOL * cg + 16 * c + m;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[kb][i] = S0 ? S0[sb + (size_t)(16 * kb + 4 * g + i) * DV + scol] : 0.f;

    // Transposed V reads (ds_read_b64_tr_b16): in each 16-lane group, lane
    // 4i + q supplies the address of 4 consecutive 16-bit values -- columns
    // 4q .. 4q+3 of row i of a 4 x 16 block -- and lane j receives column j of
    // the 4 rows.  Lane (g, m) points at row 16r + 4g + m/4, columns
    // 16c + 4(m%4) .. +3 of the V tile and receives V[16r + 4g + i][16c + m].
    int vt_off[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 16 * r + 4 * g + (m >> 2), cc = 16 * c + 4 * (m & 3);
        const int piece = (cc / CF::VEPS) ^ ((row >> 2) & (CF::VSPR - 1));
        vt_off[r] = (row * NCOL + piece * CF::VEPS + cc % CF::VEPS) * (int)sizeof(TIn);
    }

    // K^T operands of the state update from the K image, by transposed reads:
    // the A operand of pair (kb, qq) holds K[32qq + 16h + 4g + i][16kb + m]
    // (h = 0, 1; i = 0..3), so lane (g, m) points at image row
    // 32qq + 16h + 4g + m/4, logical columns 16kb + 4(m%4) .. +3 -- 4 values
    // that perm_col keeps adjacent, at group 4(kb/2) + m%4, element 4(kb%2).
    // Rows differ between (qq, h) only by multiples of 16, which leave the
    // swizzle unchanged: one address per kb, the row steps are immediate
    // offsets.
    int kt_off[NKB];
    {
        const int row = 4 * g + (m >> 2);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const int grp = (4 * (kb >> 1) + (m & 3)) ^ img_swz<false>(row, DK);
            kt_off[kb] = (row * DK + grp * 8 + 4 * (kb & 1)) * 2;
        }
    }

    // Operands of chunk n (K, V, gamma, gamma_C, Ae; for the channel-wise decay
    // Et, Z, A), read one chunk ahead, spread over chunk n-1's state update
    // (after the barrier that publishes chunk n): NRD separate reads.  (The
    // channel-wise e^{G_C} per state row is read in phase B, where it is used.)
    h8 kf[NKQ][4];
    s4 vt[4], wt[4];  // V and (channel-wise decay) write-logit columns
    f4 ga[4];  // gamma of rows 16r + 4g + i (scalar decay)
    float gC;  // gamma_C (scalar decay)
    h8 afr[NPAIR];
    constexpr int NRD = 4 * NKQ + 4 + (G2 ? 4 : 4 + 1) + NPAIR;
    auto read_item = [&](int sbi, int it) {  // sbi: state buffer of the chunk
        const char *base = smem + CF::OFF_S + sbi * CF::S_BUF;
        const float *Tq = reinterpret_cast<const float *>(base + CF::S_TK);
        if (it < 4 * NKQ) {
            kf[it / 4][it % 4] = img_h8(reinterpret_cast<const E *>(base + CF::S_K), DK, 16 * (it % 4) + m, it / 4, g);
        } else if ((it -= 4 * NKQ) < 4) {
            vt[it] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(base + CF::S_V + vt_off[it]));
        } else if (G2) {
            if ((it -= 4) < 4) {
                wt[it] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(base + CF::S_W + vt_off[it]));
            } else {
                it -= 4;
                afr[it] = *reinterpret_cast<const h8 *>(reinterpret_cast<const E *>(base + CF::S_A) + lane * 8 + it * 512);
            }
        } else if ((it -= 4) < 4) {
            ga[it] = *reinterpret_cast<const f4 *>(Tq + 16 * it + 4 * g);
        } else if ((it -= 4) < 1) {
            gC = Tq[C - 1];
        } else {
            it -= 1;
            afr[it] = *reinterpret_cast<const h8 *>(reinterpret_cast<const E *>(base + CF::S_A) + lane * 8 + it * 512);
        }
    };

    // Instruction schedule.  Within one wave, LDS accesses and vector
    // arithmetic hardly overlap each other, while a matrix product overlaps
    // both if independent work is issued right behind it; the compiler, left
    // alone, groups the products (and issues LDS reads just before their use).
    // So each phase is a sequence of fenced steps: one product plus the
    // independent vector / LDS work that fits under it.
    //   A  P = K S (4 NKQ products)     | S operand pairs and their hand-over,
    //                                     K^T reads
    //   B  Ae R' (6 products)           | R' = V - gamma P and its hand-over,
    //                                     decay of S
    //   -- barrier: chunk n+1 is staged, this chunk's buffer is released
    //   E  S += K^T (eta Delta)         | next chunk's operand reads
    //      (4 NKQ products)
#define GDN_STEP() __builtin_amdgcn_sched_barrier(0)
    constexpr int NSTEP = 4 * NKQ;  // products in phase A (and in E)

    bare_barrier();  // P(-1): chunk 0 staged
    if (NC > 0) {
#pragma unroll
        for (int it = 0; it < NRD; ++it) read_item(0, it);
    }
    int cur = 0;  // state buffer of chunk n
    for (int n = 0; n < NC; ++n) {
        const int nxt = cur == CF::NSB - 1 ? 0 : cur + 1;
        const char *Ks8 = smem + CF::OFF_S + cur * CF::S_BUF + CF::S_KH;  // K^T operands (Kh for the channel-wise decay)
        char *xb = smem + CF::OFF_X;
        // K^T operand pair (kb, qq): two transposed reads, rows 32qq and 32qq + 16 on
        auto kt_pair = [&](int kb, int qq) {
            const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(Ks8 + kt_off[kb] + 32 * qq * DK * 2));
            const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(Ks8 + kt_off[kb] + (32 * qq + 16) * DK * 2));
            return cat_h8(__builtin_bit_cast(h4, lo), __builtin_bit_cast(h4, hi));
        };
        auto sp_pair = [&](int kq) { return cat_h8(to_h4(S[2 * kq]), to_h4(S[2 * kq + 1])); };
        // S rows 16kb .. 16kb+15 decay to the chunk end: by gamma_C, or per
        // key channel by e^{G_C} (state rows 16kb + 4g + i)
        f4 gcv[NKB];
        if constexpr (G2) {
            const float *Tq = reinterpret_cast<const float *>(smem + CF::OFF_S + cur * CF::S_BUF + CF::S_TK);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) gcv[kb] = *reinterpret_cast<const f4 *>(Tq + 16 * kb + 4 * g);
        }
        auto decay = [&](int kb) {
            if constexpr (G2) S[kb] = S[kb] * gcv[kb];
            else S[kb] *= gC;
        };
        h8 Sp[NKQ];
        h8 tf[NKB][2];
        f4 P[4], Ae[4];
        h4 Rb[4], De[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) P[r] = Ae[r] = f4{0, 0, 0, 0};
        // residual of row tile rr: R' = V - gamma P in float32, then float16
        // (row tiles 2q, 2q+1 form operand pair q, handed over as one 1 KB block)
        auto resid = [&](int rr) {
            f4 x;
            if constexpr (G2) {  // z - Et S with z = sigmoid(write) v (bfloat16 inputs)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    x[i] = bf16_to_f32((uint16_t)vt[rr][i]) * sigmoid_fast(bf16_to_f32((uint16_t)wt[rr][i]));
                Rb[rr] = to_h4(x - P[rr]);
            } else {  // V (bfloat16) - gamma K S
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = bf16_to_f32((uint16_t)vt[rr][i]);
                Rb[rr] = to_h4(x - ga[rr] * P[rr]);
            }
            if (rr & 1)
                *reinterpret_cast<h8 *>(xb + CF::X_R + (c * 2 + rr / 2) * 1024 + lane * 16) = cat_h8(Rb[rr - 1], Rb[rr]);
        };

        // ---- A
        Sp[0] = sp_pair(0);
        GDN_STEP();
#pragma unroll
        for (int j = 0; j < NSTEP; ++j) {
            const int kq = j / 4, r = j % 4;
            P[r] = mfma_f16_k32(kf[kq][r], Sp[kq], P[r]);
            if (r == 0 && kq + 1 < NKQ) Sp[kq + 1] = sp_pair(kq + 1);
            if (r == 1) *reinterpret_cast<h8 *>(xb + CF::X_S + (c * NKQ + kq) * 1024 + lane * 16) = Sp[kq];
            tf[j / 2][j % 2] = kt_pair(j / 2, j % 2);
            GDN_STEP();
        }
        // ---- B: Ae R' in the order (r, q) = (0,0) (1,0) (2,0) (3,0) (2,1) (3,1)
        resid(0);
        resid(1);
        GDN_STEP();
        Ae[0] = mfma_f16_k32(afr[pair_index(0, 0)], cat_h8(Rb[0], Rb[1]), Ae[0]);
        resid(2);
        GDN_STEP();
        Ae[1] = mfma_f16_k32(afr[pair_index(1, 0)], cat_h8(Rb[0], Rb[1]), Ae[1]);
        resid(3);
        GDN_STEP();
        Ae[2] = mfma_f16_k32(afr[pair_index(2, 0)], cat_h8(Rb[0], Rb[1]), Ae[2]);
        decay(0);
        decay(1);
        De[0] = to_h4(Ae[0]);
        GDN_STEP();
        Ae[3] = mfma_f16_k32(afr[pair_index(3, 0)], cat_h8(Rb[0], Rb[1]), Ae[3]);
        decay(2);
        decay(3);
        De[1] = to_h4(Ae[1]);
        GDN_STEP();
        Ae[2] = mfma_f16_k32(afr[pair_index(2, 1)], cat_h8(Rb[2], Rb[3]), Ae[2]);
#pragma unroll
        for (int kb = 4; kb < NKB; ++kb) decay(kb);
        GDN_STEP();
        Ae[3] = mfma_f16_k32(afr[pair_index(3, 1)], cat_h8(Rb[2], Rb[3]), Ae[3]);

        // every LDS access to this chunk's inputs is complete (its operands are
        // in registers) and the hand-over is written: P(n) publishes the
        // hand-over and lets the loaders refill this chunk's buffer
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        bare_barrier();
        De[2] = to_h4(Ae[2]);
        De[3] = to_h4(Ae[3]);
        GDN_STEP();

        // ---- E: S = gamma_C S + K^T (eta Delta); the next chunk's operand
        //      reads are spread between the products (after the last chunk
        //      they read a released buffer, in bounds, and go unused)
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            const int kb = st / 2, qq = st % 2;
            S[kb] = mfma_f16_k32(tf[kb][qq], cat_h8(De[2 * qq], De[2 * qq + 1]), S[kb]);
#pragma unroll
            for (int it = 0; it < NRD; ++it)
                if (it * NSTEP / NRD == st) read_item(nxt, it);
            GDN_STEP();
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        bare_barrier();  // F(n): the output waves have read the hand-over
        cur = nxt;
    }
#undef GDN_STEP

    if (ST) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) ST[sb + (size_t)(16 * kb + 4 * g + i) * DV + scol] = S[kb][i];
    }
}

// T == 0: the final state is the initial state (or zero).
__global__ void state_copy_kernel(size_t n, const float *__restrict__ S0, float *__restrict__ ST) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        ST[i] = S0 ? S0[i] : 0.f;
}

template <bool F32, typename TIn, int DK, int DV>
static hipError_t launch_scan_t(const PrefillArgs &p, const PrefillWorkspace &ws, hipStream_t s) {
    typedef typename mma<F32>::E E;
    if constexpr (!F32) {
        constexpr int NL = 2;
        const int NC = (p.T + C - 1) / C;
        // 32 columns per work-group while that gives at most two work-groups per
        // CU; beyond, 64 columns (four state waves, one per SIMD), so that all
        // chains run in one round instead of two
        static int cus = 0;
        if (cus == 0) {
            int dev = 0, n = 0;
            if (hipGetDevice(&dev) == hipSuccess &&
                hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
                cus = n;
            else
                cus = 256;
        }
        const long long units32 = (long long)p.B * p.Hv * (DV / 32);
        if (units32 > cus) {
            typedef SplitCfg<TIn, DK, NL, false, 4> CF4;
            const unsigned blocks = (unsigned)(p.B * p.Hv * (DV / CF4::NCOL));
            hipLaunchKernelGGL((scan_split_kernel<TIn, DK, DV, NL, false, 4>), dim3(blocks), dim3(64 * (4 + 2 + NL)),
                               0, s, p.T, p.Hk, p.Hv, NC, p.v, (const void *)nullptr, ws.tok, (const E *)ws.apair,
                               (const E *)ws.qpair,
                               (const E *)ws.qimg, (const E *)ws.kimg, (const E *)nullptr, (const float *)nullptr,
                               p.S0, (TIn *)p.out, p.ST);
        } else {
            const unsigned blocks = (unsigned)(p.B * p.Hv * (DV / SplitCfg<TIn, DK, NL, false, 2>::NCOL));
            hipLaunchKernelGGL((scan_split_kernel<TIn, DK, DV, NL, false, 2>), dim3(blocks), dim3(64 * (2 + 2 + NL)),
                               0, s, p.T, p.Hk, p.Hv, NC, p.v, (const void *)nullptr, ws.tok, (const E *)ws.apair,
                               (const E *)ws.qpair,
                               (const E *)ws.qimg, (const E *)ws.kimg, (const E *)nullptr, (const float *)nullptr,
                               p.S0, (TIn *)p.out, p.ST);
        }
        return hipGetLastError();
    } else {
        constexpr int NW = 2, NL = 2;
        const int NC = (p.T + C - 1) / C;
        const unsigned blocks = (unsigned)(p.B * p.Hv * (DV / (16 * NW)));
        hipLaunchKernelGGL((state_scan_kernel<F32, TIn, DK, DV, NW, NL>), dim3(blocks), dim3(64 * (NW + NL)), 0, s,
                           p.T, p.Hk, p.Hv, NC, (const TIn *)p.v, ws.tok, (const E *)ws.apair,
                           (const E *)ws.qpair, (const E *)ws.qimg, (const E *)ws.kimg, (const E *)ws.timg,
                           p.S0, (TIn *)p.out, p.ST);
        return hipGetLastError();
    }
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

// Gated DeltaNet-2 (channel-wise decay, bfloat16 inputs): the same work-group
// with Et for P, Kh for the state update, Z for V, e^{G_C} per state row.
template <int DK, int DV>
static hipError_t launch_scan2_t(const Gdn2Args &p, const Gdn2Workspace &ws, hipStream_t s) {
    constexpr int NL = 2;
    const int NC = (p.T + C - 1) / C;
    const unsigned blocks = (unsigned)(p.B * p.Hv * (DV / SplitCfg<bf16_t, DK, NL, true, 2>::NCOL));
    hipLaunchKernelGGL((scan_split_kernel<bf16_t, DK, DV, NL, true, 2>), dim3(blocks), dim3(64 * (2 + 2 + NL)), 0, s,
                       p.T, p.Hk, p.Hv, NC, p.v, p.write, (const float *)nullptr,
                       (const _Float16 *)ws.apair, (const _Float16 *)ws.qpair, (const _Float16 *)ws.qimg,
                       (const _Float16 *)ws.eimg, (const _Float16 *)ws.khimg, ws.gc, p.S0, (bf16_t *)p.out, p.ST);
    return hipGetLastError();
}

// float32 inputs: the float32 scan with the channel-wise decay
template <int DK, int DV>
static hipError_t launch_scan2_f32_t(const Gdn2Args &p, const Gdn2Workspace &ws, hipStream_t s) {
    constexpr int NW = 2, NL = 2;
    const int NC = (p.T + C - 1) / C;
    const unsigned blocks = (unsigned)(p.B * p.Hv * (DV / (16 * NW)));
    hipLaunchKernelGGL((state_scan_kernel<true, float, DK, DV, NW, NL, true>), dim3(blocks), dim3(64 * (NW + NL)), 0, s,
                       p.T, p.Hk, p.Hv, NC, (const float *)ws.z, ws.gc, (const float *)ws.apair,
                       (const float *)ws.qpair, (const float *)ws.qimg, (const float *)ws.eimg,
                       (const float *)ws.khtimg, p.S0, (float *)p.out, p.ST);
    return hipGetLastError();
}

hipError_t launch_state_scan2(const Gdn2Args &p, const Gdn2Workspace &ws, hipStream_t s) {
    if (p.f32) {
        if (p.Dk == 128 && p.Dv == 128) return launch_scan2_f32_t<128, 128>(p, ws, s);
        if (p.Dk == 128 && p.Dv == 64) return launch_scan2_f32_t<128, 64>(p, ws, s);
        if (p.Dk == 64 && p.Dv == 128) return launch_scan2_f32_t<64, 128>(p, ws, s);
        if (p.Dk == 64 && p.Dv == 64) return launch_scan2_f32_t<64, 64>(p, ws, s);
        return hipErrorInvalidValue;
    }
    if (p.Dk == 128 && p.Dv == 128) return launch_scan2_t<128, 128>(p, ws, s);
    if (p.Dk == 128 && p.Dv == 64) return launch_scan2_t<128, 64>(p, ws, s);
    if (p.Dk == 64 && p.Dv == 128) return launch_scan2_t<64, 128>(p, ws, s);
    if (p.Dk == 64 && p.Dv == 64) return launch_scan2_t<64, 64>(p, ws, s);
    return hipErrorInvalidValue;
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
