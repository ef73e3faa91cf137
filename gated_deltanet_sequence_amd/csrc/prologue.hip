// prologue.hip -- depthwise causal convolution over time (kernel 4) + SiLU over
// the mixed q|k|v projection, written out as the separate q, k, v tensors the
// core takes (dingfen.github.io, section 10: x -> Linear -> CausalConv1D ->
// SiLU -> q, k, v; 10100.com: kernel size 4; wanger-sjtu Qwen3.5 GDN page: a
// depthwise causal conv over the mixed QKV channels whose inputs are cached
// for decode).  Per sequence b, channel c, token t:
//     y[b,t,c] = act(bias[c] + sum_{j<K} w[c][j] x[b, t-K+1+j, c]),
// inputs before token 0 from the cached state [B][K-1][C] (or zero).
// A streaming kernel (about a dozen flops per 4 bytes moved): a thread owns
// 4 channels (8-byte accesses for bfloat16, 16-byte for float32, non-temporal
// stores) of CONV_TT consecutive tokens, issues all CONV_TT + K - 1 row loads
// (its outputs plus the K-1 halo) before any arithmetic and keeps the window in
// registers.  Four channels rather than eight keep a thread at ~72 registers, so
// seven waves share a SIMD and one wave's arithmetic overlaps the others'
// loads; at eight channels (~140 registers, three waves) the SiLU's issue time
// showed through.  The new state (the last K-1 inputs) is written by the first
// token block's threads, which are also the only readers of the old state:
// in-place state update is race-free.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

constexpr int CONV_TT = 16;  // tokens per thread
constexpr int CONV_CH = 4;   // channels per thread

template <typename T> struct Row4;
template <> struct Row4<bf16_t> {
    typedef u16x4 raw;
    __device__ static __forceinline__ raw zero() { return u16x4{0, 0, 0, 0}; }
    __device__ static __forceinline__ raw ld(const void *p, size_t i) {
        return *reinterpret_cast<const u16x4 *>(static_cast<const uint16_t *>(p) + i);
    }
    __device__ static __forceinline__ void st(void *p, size_t i, raw r) {  // written once: non-temporal
        __builtin_nontemporal_store(r, reinterpret_cast<u16x4 *>(static_cast<uint16_t *>(p) + i));
    }
    __device__ static __forceinline__ float get(const raw &r, int j) { return bf16_to_f32(r[j]); }
    __device__ static __forceinline__ void st_f(void *p, size_t i, const float (&y)[4]) {
        st(p, i, u16x4{f32_to_bf16(y[0]), f32_to_bf16(y[1]), f32_to_bf16(y[2]), f32_to_bf16(y[3])});
    }
};
template <> struct Row4<float> {
    typedef f4 raw;
    __device__ static __forceinline__ raw zero() { return f4{0, 0, 0, 0}; }
    __device__ static __forceinline__ raw ld(const void *p, size_t i) {
        return *reinterpret_cast<const f4 *>(static_cast<const float *>(p) + i);
    }
    __device__ static __forceinline__ void st(void *p, size_t i, raw r) {
        __builtin_nontemporal_store(r, reinterpret_cast<f4 *>(static_cast<float *>(p) + i));
    }
    __device__ static __forceinline__ float get(const raw &r, int j) { return r[j]; }
    __device__ static __forceinline__ void st_f(void *p, size_t i, const float (&y)[4]) {
        st(p, i, f4{y[0], y[1], y[2], y[3]});
    }
};

template <typename E, int K, bool SILU>
__global__ __launch_bounds__(256) void causal_conv1d_kernel(ConvArgs p) {
    typedef Row4<E> R4;
    constexpr int W = CONV_TT + K - 1;  // rows in the window
    // bfloat16 SiLU with log2 e folded into the weights and bias: a = x log2 e
    // and x sigmoid(x) = a / (log2 e (1 + 2^-a)), one exp2, one fma, one
    // reciprocal, one multiply.  float32 keeps the exact-exponential sigmoid.
    constexpr bool FOLD = SILU && sizeof(E) == 2;
    constexpr float L2E = 1.4426950408889634f, WS = FOLD ? L2E : 1.f;
    const int cg = blockIdx.x * 256 + threadIdx.x;
    if (cg * CONV_CH >= p.C) return;  // no barriers below
    const int c0 = cg * CONV_CH, b = blockIdx.z, t0 = blockIdx.y * CONV_TT, T = p.T, C = p.C;
    const void *state = p.state;
    // interior token blocks (the window inside [0, T), all outputs < T) take
    // straight-line loads and stores from one base offset; a per-row test with
    // the cached-state fallback put several scalar branches in front of every
    // load and cut the bytes in flight
    const bool interior = t0 >= K - 1 && t0 + CONV_TT <= T;
    typename R4::raw win[W];
    if (interior) {
        const size_t base = ((size_t)b * T + (t0 - (K - 1))) * C + c0;
#pragma unroll
        for (int i = 0; i < W; ++i) win[i] = R4::ld(p.x, base + (size_t)i * C);
    } else {
#pragma unroll
        for (int i = 0; i < W; ++i) {
            const int s = t0 - (K - 1) + i;  // input token of window row i
            win[i] = R4::zero();
            if (s >= 0 && s < T) win[i] = R4::ld(p.x, ((size_t)b * T + s) * C + c0);
            else if (s < 0 && state) win[i] = R4::ld(state, ((size_t)b * (K - 1) + (K - 1 + s)) * C + c0);
        }
    }
    // weights and bias after the window, with no branch around a load: a
    // guarded load's wait would also wait for every window row issued before it
    const f4 *wp = reinterpret_cast<const f4 *>(p.w + (size_t)c0 * K);
    const float *bp = p.bias ? p.bias : p.w;  // any valid address when there is no bias
    const bool has_bias = p.bias != nullptr;
    float w[CONV_CH][K], bias[CONV_CH];
#pragma unroll
    for (int j = 0; j < CONV_CH; ++j) {
        static_assert(K == 4, "one float4 of weights per channel");
        const f4 wj = wp[j];
#pragma unroll
        for (int k = 0; k < K; ++k) w[j][k] = wj[k] * WS;
        const float bj = bp[c0 + j];
        bias[j] = has_bias ? bj * WS : 0.f;
    }
    // destination: the q, k or v tensor that holds these channels
    void *dst;
    int cd, dw;  // channel offset within the destination row, destination row width
    if (c0 < p.qk) {
        dst = p.q; cd = c0; dw = p.qk;
    } else if (c0 < 2 * p.qk) {
        dst = p.k; cd = c0 - p.qk; dw = p.qk;
    } else {
        dst = p.v; cd = c0 - 2 * p.qk; dw = C - 2 * p.qk;
    }
    const size_t obase = ((size_t)b * T + t0) * dw + cd;
    const int nout = T - t0 < CONV_TT ? T - t0 : CONV_TT;  // outputs of this block (uniform)
    // a guarded body, not an early exit: the loop must unroll fully so that the
    // window stays in registers (a runtime exit left it in scratch memory)
#pragma unroll
    for (int i = 0; i < CONV_TT; ++i) {
        if (i < nout) {
            float y[CONV_CH];
#pragma unroll
            for (int j = 0; j < CONV_CH; ++j) {
                float acc = bias[j];
#pragma unroll
                for (int k = 0; k < K; ++k) acc += w[j][k] * R4::get(win[i + k], j);
                if (!SILU) y[j] = acc;
                else if (FOLD) y[j] = acc * __builtin_amdgcn_rcpf(__builtin_fmaf(__builtin_amdgcn_exp2f(-acc), L2E, L2E));
                else y[j] = acc * sigmoid_f32(acc);
            }
            R4::st_f(dst, obase + (size_t)i * dw, y);
        }
    }
    if (blockIdx.y == 0 && p.state_out) {
        // the last K-1 inputs; older cached inputs when T < K-1
#pragma unroll
        for (int i = 0; i < K - 1; ++i) {
            const int s = T - (K - 1) + i;
            typename R4::raw r = R4::zero();
            if (s >= 0) r = R4::ld(p.x, ((size_t)b * T + s) * C + c0);
            // cached slot K-1+s = T+i >= i: not yet overwritten when the state is updated in place
            else if (state) r = R4::ld(state, ((size_t)b * (K - 1) + (K - 1 + s)) * C + c0);
            R4::st(p.state_out, ((size_t)b * (K - 1) + i) * C + c0, r);
        }
    }
}

template <typename T, bool SILU>
static hipError_t launch_conv_t(const ConvArgs &p, hipStream_t s) {
    const dim3 grid((unsigned)((p.C / CONV_CH + 255) / 256),
                    (unsigned)(p.T > 0 ? (p.T + CONV_TT - 1) / CONV_TT : 1), (unsigned)p.B);
    hipLaunchKernelGGL((causal_conv1d_kernel<T, 4, SILU>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_causal_conv1d(const ConvArgs &p, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    if (p.K != 4 || p.C % CONV_CH || p.qk % CONV_CH) return hipErrorInvalidValue;
    if (p.f32) return p.silu ? launch_conv_t<float, true>(p, s) : launch_conv_t<float, false>(p, s);
    return p.silu ? launch_conv_t<bf16_t, true>(p, s) : launch_conv_t<bf16_t, false>(p, s);
}

int conv_tokens_per_thread() { return CONV_TT; }

}  // namespace gdn
