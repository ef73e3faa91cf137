// chunk_local2_f32.hip -- chunk-local auxiliaries of the Gated DeltaNet-2
// chunked prefill for float32 inputs (float32 matrix-core operands).
//
// The quantities are those of the bfloat16 kernel (chunk_local2.hip; zhichai.net
// "Gated DeltaNet-2" digest, sections on the decoupled erase/write update and
// "高效训练：WY 算法依然成立"): per chunk of C = 64 tokens, with G the in-chunk
// inclusive prefix of g = -exp(A_log) softplus(a) per key channel,
//   Et = e . e^{G},  Qt = scale q . e^{G},  Kh = k . e^{G_C - G}  (and Kh^T),
//   M[t][i]  = sum_c e_t[c] k_i[c] e^{G_t[c] - G_i[c]}        (i < t),
//   Aq[t][i] = sum_c scale q_t[c] k_i[c] e^{G_t[c] - G_i[c]}  (i <= t),
//   A = (I + M)^{-1},  the fragments of A and of Aq A,  e^{G_C},  z = sigmoid(write) v,
// with e = sigmoid(erase) k.  Here the decay ratios are taken pair by pair, as
// the exponential of a difference of float64 prefixes (no reference splitting):
// each ratio is then exact to float32 rounding however large |G| grows, which
// the float32 path's 1e-5 tolerance needs, and no factor exceeds 1.
//
// One work-group of 4 waves per (sequence, value head, chunk).  LDS holds G
// (float64) and e, k, scale q (float32) as [64][d_k] rows whose 16-byte groups
// are XOR-swizzled by the row: 160 KB at d_k = 128 (one work-group per CU).
#include "prefill_common.h"

namespace gdn {
namespace {

template <int DK> struct Cl2F32Cfg {
    static constexpr int FG = DK / 4;  // float4 groups per float row
    static constexpr int DG = DK / 2;  // double2 groups per double row
    static constexpr int LDS = C * DK * 8 + 3 * C * DK * 4;
    static_assert(C * DK * 8 >= 3 * 10 * 256 * 4, "M, Aq and the inverse's blocks reuse the G space");
};

// float (r, c) of a swizzled [64][DK] float array; double (r, c) of a swizzled double array
template <int DK> __device__ __forceinline__ int fsw(int r, int c) {
    return r * DK + ((((c >> 2) ^ r) & (DK / 4 - 1)) << 2) + (c & 3);
}
template <int DK> __device__ __forceinline__ int dsw(int r, int c) {
    return r * DK + ((((c >> 1) ^ r) & (DK / 2 - 1)) << 1) + (c & 1);
}
// channels c .. c+3 (c a multiple of 4) of row r
template <int DK> __device__ __forceinline__ f4 ldf4(const float *X, int r, int c) {
    return *reinterpret_cast<const f4 *>(X + fsw<DK>(r, c));
}
template <int DK> __device__ __forceinline__ void ldd4(const double *X, int r, int c, double (&x)[4]) {
    typedef double d2 __attribute__((ext_vector_type(2)));
    const d2 a = *reinterpret_cast<const d2 *>(X + dsw<DK>(r, c)), b = *reinterpret_cast<const d2 *>(X + dsw<DK>(r, c + 2));
    x[0] = a[0]; x[1] = a[1]; x[2] = b[0]; x[3] = b[1];
}

template <int DK, int DV>
__global__ __launch_bounds__(256) void chunk_local2_f32_kernel(
    int T, int Hk, int Hv, int NC, float scale, const float *__restrict__ q, const float *__restrict__ k,
    const float *__restrict__ v, const float *__restrict__ a, const float *__restrict__ erase,
    const float *__restrict__ write, const float *__restrict__ A_log, float *__restrict__ eimg,
    float *__restrict__ khimg, float *__restrict__ qimg, float *__restrict__ khtimg, float *__restrict__ apair,
    float *__restrict__ qpair, float *__restrict__ gc, float *__restrict__ z) {
    typedef Cl2F32Cfg<DK> CF;
    __shared__ __attribute__((aligned(16))) char smem[CF::LDS];
    double *Gd = reinterpret_cast<double *>(smem);  // g, then its prefix G; later M, Aq, X
    float *El = reinterpret_cast<float *>(smem + C * DK * 8), *Kl = El + C * DK, *Ql = Kl + C * DK;
    float *Ms = reinterpret_cast<float *>(smem), *Qs = Ms + 10 * 256, *Xw = Qs + 10 * 256;

    const int u = blockIdx.x;
    const int n = u % NC, hv = (u / NC) % Hv, bb = u / (NC * Hv), hk = hv / (Hv / Hk);
    const int t0 = n * C;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t vu = ((size_t)bb * Hv + hv) * NC + n;

    // ---- 1. gates and key-side rows into LDS (zero past T); z to the workspace
    for (int it = tid; it < C * CF::FG; it += 256) {
        const int r = it / CF::FG, c = (it % CF::FG) * 4, t = t0 + r;
        f4 qv = {0, 0, 0, 0}, kv = {0, 0, 0, 0}, ev = {0, 0, 0, 0};
        double gv[4] = {0, 0, 0, 0};
        if (t < T) {
            const size_t kq = (((size_t)bb * T + t) * Hk + hk) * DK + c;
            const size_t ka = (((size_t)bb * T + t) * Hv + hv) * DK + c;
            qv = *reinterpret_cast<const f4 *>(q + kq);
            kv = *reinterpret_cast<const f4 *>(k + kq);
            const f4 av = *reinterpret_cast<const f4 *>(a + ka), xv = *reinterpret_cast<const f4 *>(erase + ka);
            const f4 al = *reinterpret_cast<const f4 *>(A_log + (size_t)hv * DK + c);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                gv[j] = (double)(-expf(al[j]) * softplus_f32(av[j]));
                ev[j] = sigmoid_f32(xv[j]) * kv[j];
            }
        }
        *reinterpret_cast<f4 *>(El + fsw<DK>(r, c)) = ev;
        *reinterpret_cast<f4 *>(Kl + fsw<DK>(r, c)) = kv;
        *reinterpret_cast<f4 *>(Ql + fsw<DK>(r, c)) = scale * qv;
#pragma unroll
        for (int j = 0; j < 4; ++j) Gd[dsw<DK>(r, c + j)] = gv[j];
    }
    for (int it = tid; it < C * (DV / 4); it += 256) {
        const int r = it / (DV / 4), c = (it % (DV / 4)) * 4, t = t0 + r;
        if (t < T) {
            const size_t kv = (((size_t)bb * T + t) * Hv + hv) * DV + c;
            const f4 vv = *reinterpret_cast<const f4 *>(v + kv), wv = *reinterpret_cast<const f4 *>(write + kv);
            f4 zv;
#pragma unroll
            for (int j = 0; j < 4; ++j) zv[j] = sigmoid_f32(wv[j]) * vv[j];
            *reinterpret_cast<f4 *>(z + kv) = zv;
        }
    }
    __syncthreads();

    // ---- 2. G: inclusive prefix over the chunk's tokens, one thread per channel
    //         (float64: the ratios below are differences of these sums)
    if (tid < DK) {
        double acc = 0.0;
        for (int r = 0; r < C; ++r) {
            acc += Gd[dsw<DK>(r, tid)];
            Gd[dsw<DK>(r, tid)] = acc;
        }
        gc[vu * DK + tid] = expf((float)acc);  // e^{G_C}
    }
    __syncthreads();

    // ---- 3. images Et, Qt, Kh ([64][d_k]) and Kh^T ([d_k][64]), float32 layout
    const size_t io = vu * (size_t)C * DK;
    for (int it = tid; it < C * CF::FG; it += 256) {
        const int r = it / CF::FG, c = (it % CF::FG) * 4;
        double gt[4], gC[4];
        ldd4<DK>(Gd, r, c, gt);
        ldd4<DK>(Gd, C - 1, c, gC);
        f4 fe, fk;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            fe[j] = __expf((float)gt[j]);
            fk[j] = __expf((float)(gC[j] - gt[j]));
        }
        const int o = img_index<true>(r, DK, c);
        *reinterpret_cast<f4 *>(eimg + io + o) = fe * ldf4<DK>(El, r, c);
        *reinterpret_cast<f4 *>(qimg + io + o) = fe * ldf4<DK>(Ql, r, c);
        *reinterpret_cast<f4 *>(khimg + io + o) = fk * ldf4<DK>(Kl, r, c);
    }
    for (int it = tid; it < DK * (C / 4); it += 256) {
        const int c = it / (C / 4), r0 = (it % (C / 4)) * 4;  // channel row c, tokens r0 .. r0+3
        const double gC = Gd[dsw<DK>(C - 1, c)];
        f4 x;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = Kl[fsw<DK>(r0 + j, c)] * __expf((float)(gC - Gd[dsw<DK>(r0 + j, c)]));
        *reinterpret_cast<f4 *>(khtimg + io + img_index<true>(c, C, r0)) = x;
    }

    // ---- 4. M and Aq, pair by pair: job (row t, columns 8 cb .. 8 cb + 7),
    //         8 cb <= t; each ratio e^{G_t - G_i} from the float64 difference
    //         (clamped to <= 0: the columns past t are computed and discarded)
    constexpr int NJOB = 8 * (1 + 2 + 3 + 4 + 5 + 6 + 7 + 8);  // 288
    float mres[2][8], qres[2][8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int job = tid + 256 * h;
#pragma unroll
        for (int j = 0; j < 8; ++j) mres[h][j] = qres[h][j] = 0.f;
        if (job < NJOB) {
            // cb-major: column block cb holds rows 8 cb .. 63 (64 - 8 cb jobs)
            int cb = 0, rem = job;
            while (rem >= C - 8 * cb) rem -= C - 8 * cb++;
            const int t = 8 * cb + rem;
            for (int c = 0; c < DK; c += 4) {
                const f4 et = ldf4<DK>(El, t, c), qt = ldf4<DK>(Ql, t, c);
                double gt[4];
                ldd4<DK>(Gd, t, c, gt);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int i = 8 * cb + j;
                    const f4 ki = ldf4<DK>(Kl, i, c);
                    double gi[4];
                    ldd4<DK>(Gd, i, c, gi);
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const float f = __expf(fminf((float)(gt[s] - gi[s]), 0.f)) * ki[s];
                        mres[h][j] = fmaf(et[s], f, mres[h][j]);
                        qres[h][j] = fmaf(qt[s], f, qres[h][j]);
                    }
                }
            }
        }
    }
    __syncthreads();  // G is dead: M and Aq take its space
    {   // no job covers rows 0..7, columns 8..15 of a diagonal tile (above the diagonal): zeros
        const int d = tid / 64, e = tid % 64;
        const int o = tri_index(d, d) * 256 + (e / 8) * 16 + 8 + e % 8;
        Ms[o] = 0.f;
        Qs[o] = 0.f;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int job = tid + 256 * h;
        if (job < NJOB) {
            int cb = 0, rem = job;
            while (rem >= C - 8 * cb) rem -= C - 8 * cb++;
            const int t = 8 * cb + rem, rt = t / 16, ct = cb / 2;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = 8 * cb + j;
                const int o = tri_index(rt, ct) * 256 + (t % 16) * 16 + i % 16;
                Ms[o] = i < t ? mres[h][j] : 0.f;
                Qs[o] = i <= t ? qres[h][j] : 0.f;
            }
        }
    }
    __syncthreads();
    if (w != 0) return;

    // ---- 5. A = (I + M)^{-1} (wave 0): diagonal 16x16 blocks by forward
    //         substitution, off-diagonal blocks on the matrix cores
    f4 Lf[10];
#pragma unroll
    for (int rb = 1; rb < 4; ++rb)
#pragma unroll
        for (int kb = 0; kb < rb; ++kb)
            Lf[tri_index(rb, kb)] = *reinterpret_cast<const f4 *>(Ms + tri_index(rb, kb) * 256 + m * 16 + 4 * g);
    {
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
    inverse_offdiag<true>(Xw, Lf, m, g, xt);
    wave_lds_sync();

    // ---- 6. operand fragments of A and of Aq A (the latter from the matrix
    //         cores as (Aq A)^T = A^T Aq^T, whose accumulator is its operand layout)
    f4 aq[10];
#pragma unroll
    for (int ti = 0; ti < 10; ++ti) aq[ti] = *reinterpret_cast<const f4 *>(Qs + ti * 256 + m * 16 + 4 * g);
    float *ap = apair + vu * (NPAIR * 64 * 8) + lane * 8;
    float *qp = qpair + vu * (NPAIR * 64 * 8) + lane * 8;
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
                    for (int mb = kb; mb <= r; ++mb) acc = mma<true>::block(acc, xt[tri_index(mb, kb)], aq[tri_index(r, mb)]);
                    ov[h] = acc;
                }
            }
            const int p = pair_index(r, qq);
            *reinterpret_cast<f4 *>(ap + p * 512) = ev[0];
            *reinterpret_cast<f4 *>(ap + p * 512 + 4) = ev[1];
            *reinterpret_cast<f4 *>(qp + p * 512) = ov[0];
            *reinterpret_cast<f4 *>(qp + p * 512 + 4) = ov[1];
        }
    }
}

template <int DK, int DV>
hipError_t launch_t(const Gdn2Args &p, const Gdn2Workspace &ws, hipStream_t s) {
    const int NC = (p.T + C - 1) / C;
    const unsigned units = (unsigned)(p.B * p.Hv * NC);
    hipLaunchKernelGGL((chunk_local2_f32_kernel<DK, DV>), dim3(units), dim3(256), 0, s, p.T, p.Hk, p.Hv, NC,
                       p.scale, (const float *)p.q, (const float *)p.k, (const float *)p.v, (const float *)p.a,
                       (const float *)p.erase, (const float *)p.write, p.A_log, (float *)ws.eimg,
                       (float *)ws.khimg, (float *)ws.qimg, (float *)ws.khtimg, (float *)ws.apair,
                       (float *)ws.qpair, ws.gc, (float *)ws.z);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_local2_f32(const Gdn2Args &p, const Gdn2Workspace &ws, hipStream_t s) {
    if (p.Dk == 128 && p.Dv == 128) return launch_t<128, 128>(p, ws, s);
    if (p.Dk == 128 && p.Dv == 64) return launch_t<128, 64>(p, ws, s);
    if (p.Dk == 64 && p.Dv == 128) return launch_t<64, 128>(p, ws, s);
    if (p.Dk == 64 && p.Dv == 64) return launch_t<64, 64>(p, ws, s);
    return hipErrorInvalidValue;
}

}  // namespace gdn
