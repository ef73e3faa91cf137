// state_scan.hip -- inter-chunk state scan with fused output (method and
// notation in prefill_common.h).
//
// One work-group per (sequence, value head, NW*16 state columns); each wave owns
// 16 columns of the float32 state S[d_k][16], held in matrix-core accumulator
// tiles for the whole sequence.  The columns of S are independent recurrences
// given K, beta, gamma and A, so no data crosses waves except the staged chunk.
// Per chunk, each wave runs on the matrix cores:
//   P = K S, Qa = Q S                    (64 x d_k x 16 each)
//   Delta = R + strictly-lower(A) R,     R = beta (V - gamma P)
//   O = gamma Qa + (q.k) Delta + strictly-lower(A_qk) Delta
//   S = gamma_C S + K^T (eta Delta)      (d_k x 64 x 16)
// The accumulator tiles of S, R and Delta are the B operands of the next
// product directly (see gdn_device.h), so the state never leaves registers.
//
// Staging costs no vector ALU work: the Q, K and K^T tile images written by the
// chunk-local kernel, this group's V columns and the token records are copied
// into LDS with direct-to-LDS loads (16 bytes per lane), double-buffered one
// chunk ahead, with one barrier per chunk.  V is read and the output written
// through buffer resources bounded at the sequence end, so the ragged last
// chunk reads zeros and drops its stores with no branches.  The A / A_qk
// operand fragments are staged the same way.  Work-groups that share a key
// head are numbered consecutively and mapped onto the same XCD, so their
// common image reads hit one L2.
#include "prefill_common.h"

namespace gdn {

typedef __attribute__((address_space(3))) void lds_void_t;

template <bool F32, typename TIn, int DK, int NW>
struct ScanCfg {
    typedef typename mma<F32>::E E;
    static constexpr int NT = 64 * NW;                       // threads
    static constexpr int NCOL = 16 * NW;                     // state columns per work-group
    static constexpr size_t IMG_BYTES = (size_t)C * DK * sizeof(E);
    static constexpr int VSPR = NCOL * (int)sizeof(TIn) / 16; // 16-byte slots per V row
    static constexpr int VEPS = 16 / (int)sizeof(TIn);       // elements per V slot
    static constexpr size_t OFF_Q = 0;
    static constexpr size_t OFF_K = OFF_Q + IMG_BYTES;
    static constexpr size_t OFF_T = OFF_K + IMG_BYTES;
    static constexpr size_t OFF_V = OFF_T + IMG_BYTES;
    static constexpr size_t OFF_TK = OFF_V + (size_t)C * NCOL * sizeof(TIn);
    static constexpr size_t FRAG_BYTES = (size_t)NPAIR * 64 * 8 * sizeof(E);
    static constexpr size_t OFF_AF = OFF_TK + (size_t)C * 16;
    static constexpr size_t OFF_QF = OFF_AF + FRAG_BYTES;
    static constexpr size_t BUF = OFF_QF + FRAG_BYTES;
    static constexpr int NBUF = (2 * BUF <= 160 * 1024) ? 2 : 1;
    static constexpr int IMG_UNITS = (int)(IMG_BYTES / 1024);   // 1 KB wave copies per image
    static constexpr int V_UNITS = C * NCOL * (int)sizeof(TIn) / 1024;
    static constexpr int FRAG_UNITS = (int)(FRAG_BYTES / 1024);
    static_assert(IMG_BYTES % 1024 == 0 && (C * NCOL * sizeof(TIn)) % 1024 == 0, "copy units");
    static_assert(IMG_UNITS % NW == 0 && V_UNITS % NW == 0 && FRAG_UNITS % NW == 0, "copy split");
    static_assert(VSPR >= 4 && (VSPR & (VSPR - 1)) == 0, "V slots");
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

__device__ __forceinline__ void store_out(__amdgpu_buffer_rsrc_t r, int off_elems, float x, float *) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, x), r, off_elems * 4, 0, 0);
}
__device__ __forceinline__ void store_out(__amdgpu_buffer_rsrc_t r, int off_elems, float x, bf16_t *) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)x), r, off_elems * 2, 0, 0);
}

template <bool F32, typename TIn, int DK, int DV, int NW>
__global__ __launch_bounds__(64 * NW) void state_scan_kernel(
    int T, int Hk, int Hv, int NC, float scale, const TIn *__restrict__ v,
    const float *__restrict__ tok, const typename mma<F32>::E *__restrict__ apair,
    const typename mma<F32>::E *__restrict__ qpair, const typename mma<F32>::E *__restrict__ qimg,
    const typename mma<F32>::E *__restrict__ kimg, const typename mma<F32>::E *__restrict__ timg,
    const float *__restrict__ S0, TIn *__restrict__ out, float *__restrict__ ST) {
    typedef ScanCfg<F32, TIn, DK, NW> CF;
    typedef typename mma<F32>::E E;
    typedef typename mma<F32>::V4 V4;
    constexpr int NCOL = CF::NCOL;
    constexpr int NKB = DK / 16;
    constexpr int NCG = DV / NCOL;

    __shared__ __attribute__((aligned(1024))) char smem[CF::NBUF * CF::BUF];

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
    const int lc = 16 * w + m;              // column within the group
    const int col = NCOL * cg + lc;         // state / output column

    // sequence-bounded buffer resources for V and the output
    const size_t seq_elems = (size_t)T * Hv * DV;
    const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(v + (size_t)bb * seq_elems), 0, (int)(seq_elems * sizeof(TIn)), 0x00020000);
    const __amdgpu_buffer_rsrc_t ores = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(out + (size_t)bb * seq_elems), 0, (int)(seq_elems * sizeof(TIn)), 0x00020000);

    const size_t ku0 = ((size_t)bb * Hk + hk) * NC;   // key-head chunk units
    const size_t vu0 = ((size_t)bb * Hv + hv) * NC;   // value-head chunk units

    // ---- staging of chunk n into LDS buffer `buf` (direct-to-LDS, 1 KB per wave
    //      instruction; every address part but lane*16 is wave-uniform)
    const char *gq0 = reinterpret_cast<const char *>(qimg + ku0 * C * DK);
    const char *gk0 = reinterpret_cast<const char *>(kimg + ku0 * C * DK);
    const char *gt0 = reinterpret_cast<const char *>(timg + ku0 * C * DK);
    const char *ga0 = reinterpret_cast<const char *>(apair + vu0 * (NPAIR * 64 * 8));
    const char *gf0 = reinterpret_cast<const char *>(qpair + vu0 * (NPAIR * 64 * 8));
    const char *gtk0 = reinterpret_cast<const char *>(tok + vu0 * C * 4);
    auto stage = [&](int n, int buf) {
        char *base = smem + (size_t)buf * CF::BUF;
        const size_t io = (size_t)n * CF::IMG_BYTES, fo = (size_t)n * CF::FRAG_BYTES;
#pragma unroll
        for (int i = 0; i < CF::IMG_UNITS / NW; ++i) {
            const int u = (w + NW * i) * 1024;
            __builtin_amdgcn_global_load_lds(gq0 + io + u + lane * 16, (lds_void_t *)(base + CF::OFF_Q + u), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(gk0 + io + u + lane * 16, (lds_void_t *)(base + CF::OFF_K + u), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(gt0 + io + u + lane * 16, (lds_void_t *)(base + CF::OFF_T + u), 16, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < CF::FRAG_UNITS / NW; ++i) {
            const int u = (w + NW * i) * 1024;
            __builtin_amdgcn_global_load_lds(ga0 + fo + u + lane * 16, (lds_void_t *)(base + CF::OFF_AF + u), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(gf0 + fo + u + lane * 16, (lds_void_t *)(base + CF::OFF_QF + u), 16, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < CF::V_UNITS / NW; ++i) {
            // V slot (row, sl) of this lane; slot sl holds piece sl ^ ((row >> 2) & (VSPR-1))
            const int slot = (w + NW * i) * 64 + lane;
            const int row = slot / CF::VSPR, sl = slot % CF::VSPR;
            const int piece = sl ^ ((row >> 2) & (CF::VSPR - 1));
            const int voff = ((n * C + row) * Hv + hv) * DV + NCOL * cg + piece * CF::VEPS;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vres, (lds_void_t *)(base + CF::OFF_V + (w + NW * i) * 1024), 16,
                                                     voff * (int)sizeof(TIn), 0, 0, 0);
        }
        if (w == NW - 1)
            __builtin_amdgcn_global_load_lds(gtk0 + (size_t)n * C * 16 + lane * 16, (lds_void_t *)(base + CF::OFF_TK),
                                             16, 0, 0);
    };

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
    // output element offset of (row 4g + i of the chunk, col) relative to the sequence
    const int o_lane = (4 * g * Hv + hv) * DV + col;
    // V element (row, lc) inside the staged tile
    auto v_index = [&](int row) {
        const int piece = lc / CF::VEPS;
        return row * NCOL + ((piece ^ ((row >> 2) & (CF::VSPR - 1))) * CF::VEPS) + lc % CF::VEPS;
    };

    stage(0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): staged data has landed in LDS
    __syncthreads();

    for (int n = 0; n < NC; ++n) {
        const bool more = n + 1 < NC;
        if (more && CF::NBUF == 2) stage(n + 1, (n + 1) & 1);
        const char *base = smem + (size_t)(n % CF::NBUF) * CF::BUF;
        const E *Qs = reinterpret_cast<const E *>(base + CF::OFF_Q);
        const E *Ks = reinterpret_cast<const E *>(base + CF::OFF_K);
        const E *Kt = reinterpret_cast<const E *>(base + CF::OFF_T);
        const TIn *Vs = reinterpret_cast<const TIn *>(base + CF::OFF_V);
        const f4 *Tk = reinterpret_cast<const f4 *>(base + CF::OFF_TK);
        const E *Af = reinterpret_cast<const E *>(base + CF::OFF_AF) + lane * 8;
        const E *Qf = reinterpret_cast<const E *>(base + CF::OFF_QF) + lane * 8;

        V4 Sb[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) Sb[kb] = mma<F32>::from_f4(S[kb]);

        // ---- P = K S, Qa = Q S
        f4 P[4], Qa[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            f4 pa = {0, 0, 0, 0}, qa = {0, 0, 0, 0};
#pragma unroll
            for (int kq = 0; kq < DK / 32; ++kq) {
                V4 a0, a1;
                img_pair<F32>(Ks, DK, 16 * r + m, kq, g, a0, a1);
                pa = mma<F32>::pair(pa, a0, a1, Sb[2 * kq], Sb[2 * kq + 1]);
                img_pair<F32>(Qs, DK, 16 * r + m, kq, g, a0, a1);
                qa = mma<F32>::pair(qa, a0, a1, Sb[2 * kq], Sb[2 * kq + 1]);
            }
            P[r] = pa;
            Qa[r] = qa;
        }

        // ---- R = beta (V - gamma P)
        f4 R[4];
        V4 Rb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * r + 4 * g + i;
                const f4 tr = Tk[row];
                R[r][i] = tr[0] * (lds_in(Vs + v_index(row)) - tr[1] * P[r][i]);
            }
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
                V4 a0, a1;
                ld_pair<F32>(Af + pair_index(r, qq) * 512, a0, a1);
                acc = mma<F32>::pair(acc, a0, a1, Rb[2 * qq], Rb[2 * qq + 1]);
            }
            D[r] = acc;
            Db[r] = mma<F32>::from_f4(acc);
            f4 de;
#pragma unroll
            for (int i = 0; i < 4; ++i) de[i] = Tk[16 * r + 4 * g + i][2] * acc[i];
            De[r] = mma<F32>::from_f4(de);
        }

        // ---- O = gamma Qa + (q.k) Delta + strictly-lower(A_qk) Delta
        const int o_chunk = n * C * Hv * DV + o_lane;
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
                V4 a0, a1;
                ld_pair<F32>(Qf + pair_index(r, qq) * 512, a0, a1);
                acc = mma<F32>::pair(acc, a0, a1, Db[2 * qq], Db[2 * qq + 1]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                store_out(ores, o_chunk + (16 * r + i) * Hv * DV, scale * acc[i], (TIn *)nullptr);
        }

        // ---- S = gamma_C S + K^T (eta Delta)
        const float gC = Tk[C - 1][1];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            f4 acc = gC * S[kb];
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
                V4 a0, a1;
                img_pair<F32>(Kt, C, 16 * kb + m, qq, g, a0, a1);
                acc = mma<F32>::pair(acc, a0, a1, De[2 * qq], De[2 * qq + 1]);
            }
            S[kb] = acc;
        }

        if (more && CF::NBUF == 1) {
            __syncthreads();          // every wave is done with the single buffer
            stage(n + 1, 0);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): chunk n+1 has landed in LDS
        __syncthreads();
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

template <bool F32, typename TIn, int DK, int DV>
static hipError_t launch_scan_t(const PrefillArgs &p, const PrefillWorkspace &ws, hipStream_t s) {
    typedef typename mma<F32>::E E;
    constexpr int NW = 2;
    const int NC = (p.T + C - 1) / C;
    const unsigned blocks = (unsigned)(p.B * p.Hv * (DV / (16 * NW)));
    hipLaunchKernelGGL((state_scan_kernel<F32, TIn, DK, DV, NW>), dim3(blocks), dim3(64 * NW), 0, s,
                       p.T, p.Hk, p.Hv, NC, p.scale, (const TIn *)p.v, ws.tok, (const E *)ws.apair,
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
