// decode.hip -- one-token recurrent step of the gated delta rule on a cached
// float32 state, updated in place (rainlin-net.pages.dev "Qwen3.5", section
// "GDN详解": decay, read at k, scaled difference, rank-one write, read-out;
// wanger-sjtu.github.io Qwen3.5 GDN page: the recurrent branch updates the
// cached recurrent state).
//
// Per (sequence, value head) the step is one pass over the state:
//   alpha = exp(g), g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b)
//   kv = alpha S^T k,  qs = alpha S^T q,  delta = beta (v - kv)
//   out = scale (qs + (k.q) delta)          (= S_new^T q, read from the old S)
//   S_new = alpha S + k delta^T
// so each 64 KB state (d = 128) is read once and written once: the kernel is
// bound by HBM bandwidth.  A 512-thread work-group handles one (sequence, value
// head) at a time; thread (row group rg, column quad cq) keeps Dk/RG rows x 4
// columns of the state in registers (8 rows at d = 128) between the two
// reductions and the write-back.  The work-groups are persistent (as many as
// fit on the device: with one state per work-group the registers allow 16
// waves per CU), so the loads of some work-groups stream while others reduce
// and write back; measured faster than a double-buffered 256-thread form,
// which needs twice the registers per thread and so holds half the waves.
// Loads and stores are 16 bytes per lane and whole rows per wave, and marked
// non-temporal: each state byte is touched exactly once per step.
//
// The Gated DeltaNet-2 step (zhichai.net "Gated DeltaNet-2" digest, section
// "Gated Delta Rule-2") has the same one-pass shape with per-key-channel
// weights:
//   D = exp(-exp(A_log) softplus(a)),  e = sigmoid(erase) k,  z = sigmoid(write) v
//   r = S^T (D e),  u = z - r,  out = scale (S^T (D q) + (k.q) u)   (= S_new^T q)
//   S_new = diag(D) S + k u^T
// so the same kernel runs it with the per-row weights D e and D q in place of
// k and q, the per-row decay D in place of alpha and the write gate in place
// of beta.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

// Gate inputs: the scalar decay's a, b [units] float32, A_log, dt_bias [H_v];
// the channel-wise decay's a, erase [units][DK] and write [units][DV] in the
// input type, A_log [H_v][DK] (dt_bias unused).
template <typename T, bool G2> struct DecodeGates {
    const void *a, *b, *write;
    const float *A_log, *dt_bias;
};

constexpr int DECODE_NT = 512;  // threads per work-group

template <typename T, int DK, int DV, bool G2>
__global__ __launch_bounds__(DECODE_NT) __attribute__((amdgpu_waves_per_eu(4))) void decode_kernel(int units, int Hk, int Hv, const T *__restrict__ q,
                                                     const T *__restrict__ k,
                                                     const T *__restrict__ v,
                                                     DecodeGates<T, G2> gates,
                                                     float scale, float *__restrict__ state,
                                                     T *__restrict__ out) {
    constexpr int CQ = DV / 4;      // float4 columns of a state row
    constexpr int RG = DECODE_NT / CQ;  // row groups
    constexpr int RPT = DK / RG;    // rows held per thread
    static_assert(RG * CQ == DECODE_NT && RPT * RG == DK, "tile");

    // per state row: the read weights (k and q; D e and D q for the
    // channel-wise decay), and for the channel-wise decay the written key k,
    // the decay D and the raw q (for k.q)
    __shared__ float ks[DK], qs[DK];
    __shared__ float kw[G2 ? DK : 1], dd[G2 ? DK : 1], qr[G2 ? DK : 1];
    __shared__ f4 red_k[RG][CQ], red_q[RG][CQ];
    __shared__ f4 dsh[CQ];
    __shared__ float kq_sh;

    const int tid = threadIdx.x;
    const int cq = tid % CQ, rg = tid / CQ;
    const float *__restrict__ A_log = gates.A_log;

    // state rows rg, rg+RG, ... : for a fixed i the work-group reads RG
    // consecutive rows, i.e. one contiguous RG*DV*4-byte span.
    auto load_state = [&](f4 (&s)[RPT], int unit) {
        const float *S = state + (size_t)unit * DK * DV;
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            s[i] = __builtin_nontemporal_load(
                reinterpret_cast<const f4 *>(S + (size_t)(rg + RG * i) * DV + 4 * cq));
    };
    // this head's k, q entries (threads < DK) and gate logits, into registers
    // (the channel-wise decay: thread r < DK holds row r's a, erase, A_log)
    struct Small { float k, q, a, b, al; };
    auto load_small = [&](int unit) {
        Small r = {0.f, 0.f, 0.f, 0.f, 0.f};
        const int hv = unit % Hv, hk = hv / (Hv / Hk);
        const size_t kqoff = ((size_t)(unit / Hv) * Hk + hk) * DK;
        if constexpr (G2) {
            if (tid < DK) {
                r.a = io<T>::ld(static_cast<const T *>(gates.a), (size_t)unit * DK + tid);
                r.b = io<T>::ld(static_cast<const T *>(gates.b), (size_t)unit * DK + tid);
                r.al = A_log[(size_t)hv * DK + tid];
            }
        } else {
            r.a = static_cast<const float *>(gates.a)[unit];
            r.b = static_cast<const float *>(gates.b)[unit];
        }
        if (tid < DK) {
            r.k = io<T>::ld(k, kqoff + tid);
            r.q = io<T>::ld(q, kqoff + tid);
        }
        return r;
    };

    // One head: the state is in registers, its small inputs in `sm`.
    auto step = [&](f4 (&s)[RPT], const Small &sm, int unit) {
        const int hv = unit % Hv;
        __syncthreads();  // the previous head is done with ks, qs, dsh
        float alpha = 1.f, beta = 1.f;  // scalar decay and write strength (scalar decay only)
        if constexpr (G2) {
            if (tid < DK) {  // row tid: D, e = sigmoid(erase) k, weights D e and D q
                const float D = exp_fast(-exp_fast(sm.al) * softplus_fast(sm.a));
                ks[tid] = D * sigmoid_fast(sm.b) * sm.k;
                qs[tid] = D * sm.q;
                kw[tid] = sm.k;
                dd[tid] = D;
                qr[tid] = sm.q;
            }
        } else {
            if (tid < DK) {
                ks[tid] = sm.k;
                qs[tid] = sm.q;
            }
            // gates, float32
            const float gl = -expf(A_log[hv]) * softplus_f32(sm.a + gates.dt_bias[hv]);
            alpha = expf(gl);
            beta = sigmoid_f32(sm.b);
        }
        __syncthreads();

        if (tid < 64) {  // k.q by the first wave
            const float *kk = G2 ? kw : ks, *qq = G2 ? qr : qs;
            float p = 0.f;
            for (int i = tid; i < DK; i += 64) p += kk[i] * qq[i];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) p += __shfl_xor(p, off, 64);
            if (tid == 0) kq_sh = p;
        }
        f4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + RG * i;
            pk += s[i] * ks[r];
            pq += s[i] * qs[r];
        }
        red_k[rg][cq] = pk;
        red_q[rg][cq] = pq;
        __syncthreads();

        if (tid < CQ) {
            f4 sk = red_k[0][tid], sq = red_q[0][tid];
#pragma unroll
            for (int r = 1; r < RG; ++r) {
                sk += red_k[r][tid];
                sq += red_q[r][tid];
            }
            const f4 vv = ld4(v, (size_t)unit * DV + 4 * tid);
            f4 d;
            if constexpr (G2) {  // u = sigmoid(write) v - S^T (D e)
                const f4 wl = ld4(static_cast<const T *>(gates.write), (size_t)unit * DV + 4 * tid);
#pragma unroll
                for (int j = 0; j < 4; ++j) d[j] = sigmoid_fast(wl[j]) * vv[j] - sk[j];
            } else {
                d = beta * (vv - alpha * sk);
            }
            dsh[tid] = d;
            const f4 o = scale * (alpha * sq + kq_sh * d);
            st4(out, (size_t)unit * DV + 4 * tid, o);
        }
        __syncthreads();

        float *S = state + (size_t)unit * DK * DV;
        const f4 d = dsh[cq];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + RG * i;
            f4 sn;
            if constexpr (G2) sn = dd[r] * s[i] + kw[r] * d;
            else sn = alpha * s[i] + ks[r] * d;
            __builtin_nontemporal_store(sn, reinterpret_cast<f4 *>(S + (size_t)r * DV + 4 * cq));
        }
    };

    // Persistent loop over heads.
    f4 st[RPT];
    for (int u = blockIdx.x; u < units; u += gridDim.x) {
        load_state(st, u);
        const Small sm = load_small(u);
        step(st, sm, u);
    }
}

// Resident work-groups for the persistent decode loop: enough to keep every
// CU streaming, few enough that each walks several heads.
template <typename T, int DK, int DV, bool G2>
static unsigned decode_grid(int units) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<T, DK, DV, G2>, DECODE_NT, 0) != hipSuccess ||
        cus <= 0 || per_cu <= 0)
        return (unsigned)units;
    const long long resident = (long long)cus * per_cu;
    return (unsigned)(units < resident ? units : resident);
}

template <typename T, int DK, int DV, bool G2>
static hipError_t launch_decode_t(const DecodeArgs &p, hipStream_t s) {
    const int units = p.B * p.Hv;
    const DecodeGates<T, G2> gates{p.a, p.b, p.write, p.A_log, p.dt_bias};
    hipLaunchKernelGGL((decode_kernel<T, DK, DV, G2>), dim3(decode_grid<T, DK, DV, G2>(units)), dim3(DECODE_NT), 0, s,
                       units, p.Hk, p.Hv, (const T *)p.q, (const T *)p.k, (const T *)p.v, gates, p.scale,
                       p.state, (T *)p.out);
    return hipGetLastError();
}

template <typename T, bool G2>
static hipError_t launch_decode_dt(const DecodeArgs &p, hipStream_t s) {
    if (p.Dk == 128 && p.Dv == 128) return launch_decode_t<T, 128, 128, G2>(p, s);
    if (p.Dk == 128 && p.Dv == 64) return launch_decode_t<T, 128, 64, G2>(p, s);
    if (p.Dk == 64 && p.Dv == 128) return launch_decode_t<T, 64, 128, G2>(p, s);
    if (p.Dk == 64 && p.Dv == 64) return launch_decode_t<T, 64, 64, G2>(p, s);
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs &p, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    if (p.gdn2) return p.f32 ? launch_decode_dt<float, true>(p, s) : launch_decode_dt<bf16_t, true>(p, s);
    return p.f32 ? launch_decode_dt<float, false>(p, s) : launch_decode_dt<bf16_t, false>(p, s);
}

}  // namespace gdn
