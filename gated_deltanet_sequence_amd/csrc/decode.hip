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
// bound by HBM bandwidth.  One 256-thread work-group per (sequence, value
// head); thread (row group rg, column quad cq) keeps Dk/RG rows x 4 columns of
// the state in registers between the two reductions and the write-back.
// Loads and stores are 16 bytes per lane and whole rows per wave, and marked
// non-temporal: each state byte is touched exactly once per step.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <typename T, int DK, int DV>
__global__ __launch_bounds__(256) void decode_kernel(int Hk, int Hv, const T *__restrict__ q,
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

    const int unit = blockIdx.x;  // b * Hv + hv
    const int hv = unit % Hv;
    const int bb = unit / Hv;
    const int hk = hv / (Hv / Hk);
    const int tid = threadIdx.x;
    const int cq = tid % CQ, rg = tid / CQ;
    float *S = state + (size_t)unit * DK * DV;

    // state rows rg, rg+RG, ... : for a fixed i the work-group reads RG
    // consecutive rows, i.e. one contiguous RG*DV*4-byte span.
    f4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        s[i] = __builtin_nontemporal_load(
            reinterpret_cast<const f4 *>(S + (size_t)(rg + RG * i) * DV + 4 * cq));

    const size_t kqoff = ((size_t)bb * Hk + hk) * DK;
    for (int i = tid; i < DK; i += 256) {
        ks[i] = io<T>::ld(k, kqoff + i);
        qs[i] = io<T>::ld(q, kqoff + i);
    }
    // gates, float32
    const float gl = -expf(A_log[hv]) * softplus_f32(a[unit] + dt_bias[hv]);
    const float alpha = expf(gl);
    const float beta = sigmoid_f32(b[unit]);
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

    const f4 d = dsh[cq];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        const f4 sn = alpha * s[i] + ks[r] * d;
        __builtin_nontemporal_store(sn, reinterpret_cast<f4 *>(S + (size_t)r * DV + 4 * cq));
    }
}

template <typename T, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs &p, hipStream_t s) {
    hipLaunchKernelGGL((decode_kernel<T, DK, DV>), dim3((unsigned)(p.B * p.Hv)), dim3(256), 0, s,
                       p.Hk, p.Hv, (const T *)p.q, (const T *)p.k, (const T *)p.v, p.a, p.b,
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
