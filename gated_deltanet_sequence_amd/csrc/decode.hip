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
// bound by HBM bandwidth.  A 256-thread work-group handles one (sequence, value
// head) at a time; thread (row group rg, column quad cq) keeps Dk/RG rows x 4
// columns of the state in registers between the two reductions and the
// write-back.  The work-groups are persistent (as many as fit on the device)
// and load the next head's state while they reduce and write back the
// current one, so reads and writes stream concurrently.
// Loads and stores are 16 bytes per lane and whole rows per wave, and marked
// non-temporal: each state byte is touched exactly once per step.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <typename T, int DK, int DV>
__global__ __launch_bounds__(256) void decode_kernel(int units, int Hk, int Hv, const T *__restrict__ q,
                                                     const T *__restrict__ k,
                                                     const T *__restrict__ v,
                                                     const float *__restrict__ a,
                                                     const float *__restrict__ b,
                                                     const float *__restrict__ A_log,
                                                     const float *__restrict__ dt_bias,
                                                     float scale, float *__restrict__ state,
                                                     T *__restrict__ out) {
    constexpr int CQ = DV / 4;      // float4 columns of a state row
    constexpr int RG = 256 / CQ;    // row groups
    constexpr int RPT = DK / RG;    // rows held per thread
    static_assert(RG * CQ == 256 && RPT * RG == DK, "tile");

    __shared__ float ks[DK], qs[DK];
    __shared__ f4 red_k[RG][CQ], red_q[RG][CQ];
    __shared__ f4 dsh[CQ];
    __shared__ float kq_sh;

    const int tid = threadIdx.x;
    const int cq = tid % CQ, rg = tid / CQ;

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
    struct Small { float k, q, a, b; };
    auto load_small = [&](int unit) {
        Small r = {0.f, 0.f, a[unit], b[unit]};
        const int hv = unit % Hv, hk = hv / (Hv / Hk);
        const size_t kqoff = ((size_t)(unit / Hv) * Hk + hk) * DK;
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
        if (tid < DK) {
            ks[tid] = sm.k;
            qs[tid] = sm.q;
        }
        // gates, float32
        const float gl = -expf(A_log[hv]) * softplus_f32(sm.a + dt_bias[hv]);
        const float alpha = expf(gl);
        const float beta = sigmoid_f32(sm.b);
        __syncthreads();

        if (tid < 64) {  // k.q by the first wave
            float p = 0.f;
            for (int i = tid; i < DK; i += 64) p += ks[i] * qs[i];
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
            const f4 d = beta * (vv - alpha * sk);
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
            const f4 sn = alpha * s[i] + ks[r] * d;
            __builtin_nontemporal_store(sn, reinterpret_cast<f4 *>(S + (size_t)r * DV + 4 * cq));
        }
    };

    // Persistent loop over heads, two state buffers: the next head's state
    // is in flight while this one is reduced and written back.
    const int stride = gridDim.x;
    int u = blockIdx.x;
    if (u >= units) return;
    f4 s0[RPT], s1[RPT];
    load_state(s0, u);
    Small m0 = load_small(u), m1 = m0;
    while (true) {
        const int u1 = u + stride;
        if (u1 < units) {
            load_state(s1, u1);
            m1 = load_small(u1);
        }
        step(s0, m0, u);
        if (u1 >= units) break;
        const int u2 = u1 + stride;
        if (u2 < units) {
            load_state(s0, u2);
            m0 = load_small(u2);
        }
        step(s1, m1, u1);
        if (u2 >= units) break;
        u = u2;
    }
}

// Resident work-groups for the persistent decode loop: enough to keep every
// CU streaming, few enough that each walks several heads.
template <typename T, int DK, int DV>
static unsigned decode_grid(int units) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<T, DK, DV>, 256, 0) != hipSuccess ||
        cus <= 0 || per_cu <= 0)
        return (unsigned)units;
    const long long resident = (long long)cus * per_cu;
    return (unsigned)(units < resident ? units : resident);
}

template <typename T, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs &p, hipStream_t s) {
    const int units = p.B * p.Hv;
    hipLaunchKernelGGL((decode_kernel<T, DK, DV>), dim3(decode_grid<T, DK, DV>(units)), dim3(256), 0, s,
                       units, p.Hk, p.Hv, (const T *)p.q, (const T *)p.k, (const T *)p.v, p.a, p.b,
                       p.A_log, p.dt_bias, p.scale, p.state, (T *)p.out);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_decode_dt(const DecodeArgs &p, hipStream_t s) {
    if (p.Dk == 128 && p.Dv == 128) return launch_decode_t<T, 128, 128>(p, s);
    if (p.Dk == 128 && p.Dv == 64) return launch_decode_t<T, 128, 64>(p, s);
    if (p.Dk == 64 && p.Dv == 128) return launch_decode_t<T, 64, 128>(p, s);
    if (p.Dk == 64 && p.Dv == 64) return launch_decode_t<T, 64, 64>(p, s);
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs &p, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    return p.f32 ? launch_decode_dt<float>(p, s) : launch_decode_dt<bf16_t>(p, s);
}

}  // namespace gdn
