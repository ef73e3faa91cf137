// epilogue.hip -- gated RMS normalisation of the core's output, the step
// between the recurrence and the output projection (rainlin-net.pages.dev
// "Qwen3.5", section "GDN详解": the read-out passes through a gated RMSNorm
// with the output gate z; wanger-sjtu Qwen3.5 GDN page, section "输出门控与
// RMSNorm": the gate works like SwiGLU's; 10100.com pseudocode: a sigmoid
// gate multiplied elementwise).  Per row (one token of one value head, D
// values):
//     y = x / sqrt(mean(x^2) + eps) * w * act(z),  act = SiLU or sigmoid.
// A pure streaming kernel (read x and z, write y once: ~0.003 flop per byte),
// bound by HBM.  A row is D / 8 lanes, 8 values per lane (16-byte accesses
// for bfloat16, non-temporal); each thread issues the loads of all its rows
// before any arithmetic, then reduces the sum of squares within its lane group.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <typename T> struct V8;
template <> struct V8<bf16_t> {
    typedef u16x8 raw;
    __device__ static __forceinline__ raw ld(const bf16_t *p, size_t i) {
        return __builtin_nontemporal_load(reinterpret_cast<const u16x8 *>(reinterpret_cast<const uint16_t *>(p) + i));
    }
    __device__ static __forceinline__ float get(const raw &r, int j) { return bf16_to_f32(r[j]); }
    __device__ static __forceinline__ void st(bf16_t *p, size_t i, const float (&y)[8]) {
        u16x8 o;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = f32_to_bf16(y[j]);
        __builtin_nontemporal_store(o, reinterpret_cast<u16x8 *>(reinterpret_cast<uint16_t *>(p) + i));
    }
};
template <> struct V8<float> {
    struct raw { f4 lo, hi; };
    __device__ static __forceinline__ raw ld(const float *p, size_t i) {
        return raw{__builtin_nontemporal_load(reinterpret_cast<const f4 *>(p + i)),
                   __builtin_nontemporal_load(reinterpret_cast<const f4 *>(p + i + 4))};
    }
    __device__ static __forceinline__ float get(const raw &r, int j) { return j < 4 ? r.lo[j] : r.hi[j - 4]; }
    __device__ static __forceinline__ void st(float *p, size_t i, const float (&y)[8]) {
        __builtin_nontemporal_store(f4{y[0], y[1], y[2], y[3]}, reinterpret_cast<f4 *>(p + i));
        __builtin_nontemporal_store(f4{y[4], y[5], y[6], y[7]}, reinterpret_cast<f4 *>(p + i + 4));
    }
};

// row slots per thread, their loads issued together; with non-temporal
// accesses (each byte is touched once) 2 measured best on the prefill output's
// shape (6.0 TB/s, against 5.5 with 4 and 4.9 with 4 and cached accesses)
constexpr int NORM_ROWS_PER_THREAD = 2;

template <typename T, int D, bool SILU>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(long long rows, const T *x,
                                                            const T *__restrict__ z,
                                                            const float *__restrict__ w, float eps,
                                                            T *out) {  // out may be x (each lane reads its x before writing)
    constexpr int L = D / 8;            // lanes per row
    constexpr int RPB = 256 / L;        // rows per pass of the work-group
    constexpr int R = NORM_ROWS_PER_THREAD;
    const int tid = threadIdx.x, c8 = (tid % L) * 8;
    const long long row0 = (long long)blockIdx.x * RPB * R + tid / L;
    typename V8<T>::raw xr[R], zr[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const long long r = row0 + (long long)RPB * i;
        if (r < rows) {
            xr[i] = V8<T>::ld(x, (size_t)r * D + c8);
            zr[i] = V8<T>::ld(z, (size_t)r * D + c8);
        }
    }
    float wv[8];
    {
        const f4 a = *reinterpret_cast<const f4 *>(w + c8), b = *reinterpret_cast<const f4 *>(w + c8 + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            wv[j] = a[j];
            wv[4 + j] = b[j];
        }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const long long r = row0 + (long long)RPB * i;
        if (r >= rows) continue;  // uniform across the row's lane group
        float xv[8], ss = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            xv[j] = V8<T>::get(xr[i], j);
            ss += xv[j] * xv[j];
        }
#pragma unroll
        for (int off = L / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
        const float ms = ss * (1.f / D) + eps;
        const float inv = sizeof(T) == 4 ? 1.f / sqrtf(ms) : __builtin_amdgcn_rsqf(ms);
        float y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float zv = V8<T>::get(zr[i], j);
            const float s = sizeof(T) == 4 ? sigmoid_f32(zv) : sigmoid_fast(zv);
            y[j] = xv[j] * inv * wv[j] * (SILU ? zv * s : s);
        }
        V8<T>::st(out, (size_t)r * D + c8, y);
    }
}

template <typename T, int D, bool SILU>
static hipError_t launch_norm_t(const NormArgs &p, hipStream_t s) {
    constexpr long long per_wg = (256 / (D / 8)) * NORM_ROWS_PER_THREAD;
    const long long wgs = (p.rows + per_wg - 1) / per_wg;
    hipLaunchKernelGGL((gated_rmsnorm_kernel<T, D, SILU>), dim3((unsigned)wgs), dim3(256), 0, s, p.rows,
                       (const T *)p.x, (const T *)p.z, p.w, p.eps, (T *)p.out);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_norm_dt(const NormArgs &p, hipStream_t s) {
    if (p.d == 128) return p.silu ? launch_norm_t<T, 128, true>(p, s) : launch_norm_t<T, 128, false>(p, s);
    if (p.d == 64) return p.silu ? launch_norm_t<T, 64, true>(p, s) : launch_norm_t<T, 64, false>(p, s);
    return hipErrorInvalidValue;
}

hipError_t launch_gated_rmsnorm(const NormArgs &p, hipStream_t s) {
    if (p.rows == 0) return hipSuccess;
    return p.f32 ? launch_norm_dt<float>(p, s) : launch_norm_dt<bf16_t>(p, s);
}

// largest row count one launch takes (grid.x <= 2^31 - 1 work-groups)
long long gated_rmsnorm_max_rows() { return 16LL * NORM_ROWS_PER_THREAD * 2147483647LL; }

}  // namespace gdn
