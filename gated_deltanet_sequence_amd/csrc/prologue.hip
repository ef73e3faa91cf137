// prologue.hip -- depthwise causal convolution over time (kernel 4) + SiLU over
// the mixed q|k|v projection, written out as the separate q, k, v tensors the
// core takes (dingfen.github.io, section 10: x -> Linear -> CausalConv1D ->
// SiLU -> q, k, v; 10100.com: kernel size 4; wanger-sjtu Qwen3.5 GDN page: a
// depthwise causal conv over the mixed QKV channels whose inputs are cached
// for decode).  Per sequence b, channel c, token t:
//     y[b,t,c] = act(bias[c] + sum_{j<K} w[c][j] x[b, t-K+1+j, c]),
// inputs before token 0 from the cached state [B][K-1][C] (or zero).
// A streaming kernel (~2K flop per output, ~0.02 flop per byte): a thread owns
// 8 channels (16-byte accesses for bfloat16, non-temporal stores) of CONV_TT
// consecutive tokens,
// issues all CONV_TT + K - 1 row loads (its outputs plus the K-1 halo) before
// any arithmetic and keeps the window in registers.  The new state (the last
// K-1 inputs) is written by the first token block's threads, which are also
// the only readers of the old state: in-place state update is race-free.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

constexpr int CONV_TT = 16;  // tokens per thread

template <typename T> struct Row8;
template <> struct Row8<bf16_t> {
    typedef u16x8 raw;
    __device__ static __forceinline__ raw zero() { return u16x8{0, 0, 0, 0, 0, 0, 0, 0}; }
    __device__ static __forceinline__ raw ld(const void *p, size_t i) {
        return *reinterpret_cast<const u16x8 *>(static_cast<const uint16_t *>(p) + i);
    }
    __device__ static __forceinline__ void st(void *p, size_t i, raw r) {  // written once: non-temporal
        __builtin_nontemporal_store(r, reinterpret_cast<u16x8 *>(static_cast<uint16_t *>(p) + i));
    }
    __device__ static __forceinline__ float get(const raw &r, int j) { return bf16_to_f32(r[j]); }
    __device__ static __forceinline__ void st_f(void *p, size_t i, const float (&y)[8]) {
        u16x8 o;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = f32_to_bf16(y[j]);
        st(p, i, o);
    }
};
template <> struct Row8<float> {
    struct raw { f4 lo, hi; };
    __device__ static __forceinline__ raw zero() { return raw{f4{0, 0, 0, 0}, f4{0, 0, 0, 0}}; }
    __device__ static __forceinline__ raw ld(const void *p, size_t i) {
        const float *q = static_cast<const float *>(p) + i;
        return raw{*reinterpret_cast<const f4 *>(q), *reinterpret_cast<const f4 *>(q + 4)};
    }
    __device__ static __forceinline__ void st(void *p, size_t i, raw r) {
        float *q = static_cast<float *>(p) + i;
        __builtin_nontemporal_store(r.lo, reinterpret_cast<f4 *>(q));
        __builtin_nontemporal_store(r.hi, reinterpret_cast<f4 *>(q + 4));
    }
    __device__ static __forceinline__ float get(const raw &r, int j) { return j < 4 ? r.lo[j] : r.hi[j - 4]; }
    __device__ static __forceinline__ void st_f(void *p, size_t i, const float (&y)[8]) {
        st(p, i, raw{f4{y[0], y[1], y[2], y[3]}, f4{y[4], y[5], y[6], y[7]}});
    }
};

template <typename E, int K, bool SILU>
__global__ __launch_bounds__(256) void causal_conv1d_kernel(ConvArgs p) {
    typedef Row8<E> R8;
    constexpr int W = CONV_TT + K - 1;  // rows in the window
    const int cg = blockIdx.x * 256 + threadIdx.x;
    if (cg * 8 >= p.C) return;  // no barriers below
    const int c0 = cg * 8, b = blockIdx.z, t0 = blockIdx.y * CONV_TT, T = p.T, C = p.C;
    const void *state = p.state;
    typename R8::raw win[W];
#pragma unroll
    for (int i = 0; i < W; ++i) {
        const int s = t0 - (K - 1) + i;  // input token of window row i
        win[i] = R8::zero();
        if (s >= 0 && s < T) win[i] = R8::ld(p.x, ((size_t)b * T + s) * C + c0);
        else if (s < 0 && state) win[i] = R8::ld(state, ((size_t)b * (K - 1) + (K - 1 + s)) * C + c0);
    }
    float w[8][K], bias[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int k = 0; k < K; ++k) w[j][k] = p.w[(size_t)(c0 + j) * K + k];
        bias[j] = p.bias ? p.bias[c0 + j] : 0.f;
    }
    // destination: the q, k or v tensor that holds these 8 channels
    void *dst;
    int cd, dw;  // channel offset within the destination row, destination row width
    if (c0 < p.qk) {
        dst = p.q; cd = c0; dw = p.qk;
    } else if (c0 < 2 * p.qk) {
        dst = p.k; cd = c0 - p.qk; dw = p.qk;
    } else {
        dst = p.v; cd = c0 - 2 * p.qk; dw = C - 2 * p.qk;
    }
#pragma unroll
    for (int i = 0; i < CONV_TT; ++i) {
        const int t = t0 + i;
        if (t >= T) break;
        float y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float acc = bias[j];
#pragma unroll
            for (int k = 0; k < K; ++k) acc += w[j][k] * R8::get(win[i + k], j);
            y[j] = SILU ? acc * (sizeof(E) == 4 ? sigmoid_f32(acc) : sigmoid_fast(acc)) : acc;
        }
        R8::st_f(dst, ((size_t)b * T + t) * dw + cd, y);
    }
    if (blockIdx.y == 0 && p.state_out) {
        // the last K-1 inputs; older cached inputs when T < K-1
#pragma unroll
        for (int i = 0; i < K - 1; ++i) {
            const int s = T - (K - 1) + i;
            typename R8::raw r = R8::zero();
            if (s >= 0) r = R8::ld(p.x, ((size_t)b * T + s) * C + c0);
            // cached slot K-1+s = T+i >= i: not yet overwritten when the state is updated in place
            else if (state) r = R8::ld(state, ((size_t)b * (K - 1) + (K - 1 + s)) * C + c0);
            R8::st(p.state_out, ((size_t)b * (K - 1) + i) * C + c0, r);
        }
    }
}

template <typename T, bool SILU>
static hipError_t launch_conv_t(const ConvArgs &p, hipStream_t s) {
    const dim3 grid((unsigned)((p.C / 8 + 255) / 256), (unsigned)(p.T > 0 ? (p.T + CONV_TT - 1) / CONV_TT : 1),
                    (unsigned)p.B);
    hipLaunchKernelGGL((causal_conv1d_kernel<T, 4, SILU>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_causal_conv1d(const ConvArgs &p, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    if (p.K != 4) return hipErrorInvalidValue;
    if (p.f32) return p.silu ? launch_conv_t<float, true>(p, s) : launch_conv_t<float, false>(p, s);
    return p.silu ? launch_conv_t<bf16_t, true>(p, s) : launch_conv_t<bf16_t, false>(p, s);
}

int conv_tokens_per_thread() { return CONV_TT; }

}  // namespace gdn
