// state_scan.hip -- inter-chunk state scan with fused output (method and
// notation in prefill_common.h).
//
// One work-group per (sequence, value head, NW*16 state columns) with NW
// compute waves and NL loader waves.  Each compute wave owns 16 columns of the
// float32 state S[d_k][16], held in matrix-core accumulator tiles for the whole
// sequence; the columns of S are independent recurrences given K, beta, gamma
// and A.  Per chunk, each compute wave runs on the matrix cores:
//   P = K S, Qa = Q S                    (64 x d_k x 16 each)
//   Delta = R + strictly-lower(A) R,     R = beta (V - gamma P)
//   O = gamma Qa + (q.k) Delta + strictly-lower(A_qk) Delta
//   S = gamma_C S + K^T (eta Delta)      (d_k x 64 x 16)
// The accumulator tiles of S, R and Delta are the B operands of the next
// product directly (see gdn_device.h), so the state never leaves registers, and
// compute waves issue no global-memory instruction inside the chunk loop: the
// output tile goes to LDS.
//
// The loader waves do all global-memory traffic: while the compute waves work
// on chunk n, they copy chunk n+1 -- the Q, K and K^T tile images written by
// the chunk-local kernel, the A / A_qk operand fragments, the token records and
// this group's V columns -- into the other LDS buffer with direct-to-LDS buffer
// loads (16 bytes per lane), and write chunk n-1's output rows from LDS with
// 16-byte stores.  V and the output go through buffer resources bounded at the
// sequence end, so the ragged last chunk reads zeros and drops its stores with
// no branches.  One barrier per chunk.  Work-groups that share a key head are
// numbered consecutively and mapped onto the same XCD, so their common image
// reads hit one L2.
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

template <bool F32, typename TIn, int DK, int DV, int NW, int NL>
__global__ __launch_bounds__(64 * (NW + NL)) void state_scan_kernel(
    int T, int Hk, int Hv, int NC, const TIn *__restrict__ v,
    const float *__restrict__ tok, const typename mma<F32>::E *__restrict__ apair,
    const typename mma<F32>::E *__restrict__ qpair, const typename mma<F32>::E *__restrict__ qimg,
    const typename mma<F32>::E *__restrict__ kimg, const typename mma<F32>::E *__restrict__ timg,
    const float *__restrict__ S0, TIn *__restrict__ out, float *__restrict__ ST) {
    typedef ScanCfg<F32, TIn, DK, NW, NL> CF;
    typedef typename mma<F32>::E E;
    typedef typename mma<F32>::V4 V4;
    constexpr int NCOL = CF::NCOL;
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
        const __amdgpu_buffer_rsrc_t rq = rsrc(qimg + ku0 * C * DK, (size_t)NC * CF::IMG_BYTES);
        const __amdgpu_buffer_rsrc_t rk = rsrc(kimg + ku0 * C * DK, (size_t)NC * CF::IMG_BYTES);
        const __amdgpu_buffer_rsrc_t rt = rsrc(timg + ku0 * C * DK, (size_t)NC * CF::IMG_BYTES);
        const __amdgpu_buffer_rsrc_t ra = rsrc(apair + vu0 * (NPAIR * 64 * 8), (size_t)NC * CF::FRAG_BYTES);
        const __amdgpu_buffer_rsrc_t rf = rsrc(qpair + vu0 * (NPAIR * 64 * 8), (size_t)NC * CF::FRAG_BYTES);
        const __amdgpu_buffer_rsrc_t rtk = rsrc(tok + vu0 * C * 4, (size_t)NC * C * 16);
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
            if (l == 0)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rtk, (lds_void_t *)(base + CF::OFF_TK), 16, lane16, n * C * 16, 0, 0);
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
        const float *Tq = reinterpret_cast<const float *>(base + CF::OFF_TK);  // [beta|gamma|eta|q.k][64]
        const E *Af = reinterpret_cast<const E *>(base + CF::OFF_AF) + lane * 8;
        const E *Qf = reinterpret_cast<const E *>(base + CF::OFF_QF) + lane * 8;
        TIn *Os = reinterpret_cast<TIn *>(smem + CF::OFF_O + (size_t)(n & 1) * CF::TILE_BYTES);
        // token quantity X of this lane's rows 16r + 4g + i, i = 0..3
        auto tokq = [&](int x, int r) { return *reinterpret_cast<const f4 *>(Tq + 64 * x + 16 * r + 4 * g); };

        // operands of the residual, read ahead of the products that need them
        f4 be[4], ga[4], vv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            be[r] = tokq(0, r);
            ga[r] = tokq(1, r);
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
        f4 et[4], dq[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            et[r] = tokq(2, r);
            dq[r] = tokq(3, r);
        }

        // ---- R = beta (V - gamma P)
        f4 R[4];
        V4 Rb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            R[r] = be[r] * (vv[r] - ga[r] * P[r]);
            Rb[r] = mma<F32>::from_f4(R[r]);
        }

        // ---- Delta = R + strictly-lower(A) R
        f4 D[4];
        V4 Db[4], De[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            f4 acc = R[r];
#pragma unroll
            for (int qq = 0; qq <= r / 2; ++qq) {
                const int p = pair_index(r, qq);
                acc = mma<F32>::pair(acc, afr[p][0], afr[p][1], Rb[2 * qq], Rb[2 * qq + 1]);
            }
            D[r] = acc;
            Db[r] = mma<F32>::from_f4(acc);
            De[r] = mma<F32>::from_f4(et[r] * acc);
        }

        // K^T operands of the state update, read ahead of it
        V4 tf[NKB][2][2];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) img_pair<F32>(Kt, C, 16 * kb + m, qq, g, tf[kb][qq][0], tf[kb][qq][1]);

        // ---- O = gamma Qa + (q.k) Delta + strictly-lower(A_qk) Delta, into the
        //      LDS output tile (the read-out scale is already folded into Q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            f4 acc = ga[r] * Qa[r] + dq[r] * D[r];
#pragma unroll
            for (int qq = 0; qq <= r / 2; ++qq) {
                const int p = pair_index(r, qq);
                acc = mma<F32>::pair(acc, qfr[p][0], qfr[p][1], Db[2 * qq], Db[2 * qq + 1]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) lds_out(Os + tile_index(16 * r + 4 * g + i), acc[i]);
        }

        // ---- S = gamma_C S + K^T (eta Delta)
        const float gC = Tq[64 + C - 1];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            f4 acc = gC * S[kb];
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

// T == 0: the final state is the initial state (or zero).
__global__ void state_copy_kernel(size_t n, const float *__restrict__ S0, float *__restrict__ ST) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        ST[i] = S0 ? S0[i] : 0.f;
}

template <bool F32, typename TIn, int DK, int DV>
static hipError_t launch_scan_t(const PrefillArgs &p, const PrefillWorkspace &ws, hipStream_t s) {
    typedef typename mma<F32>::E E;
    constexpr int NW = 2, NL = 2;
    const int NC = (p.T + C - 1) / C;
    const unsigned blocks = (unsigned)(p.B * p.Hv * (DV / (16 * NW)));
    hipLaunchKernelGGL((state_scan_kernel<F32, TIn, DK, DV, NW, NL>), dim3(blocks), dim3(64 * (NW + NL)), 0, s,
                       p.T, p.Hk, p.Hv, NC, (const TIn *)p.v, ws.tok, (const E *)ws.apair,
                       (const E *)ws.qpair, (const E *)ws.qimg, (const E *)ws.kimg, (const E *)ws.timg,
                       p.S0, (TIn *)p.out, p.ST);
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
