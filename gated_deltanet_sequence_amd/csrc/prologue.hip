// prologue.hip -- depthwise causal convolution over time (kernel 4) + SiLU over
// the mixed q|k|v projection, written out as the separate q, k, v tensors the
// core takes (dingfen.github.io, section 10: x -> Linear -> CausalConv1D ->
// SiLU -> q, k, v; 10100.com: kernel size 4; wanger-sjtu Qwen3.5 GDN page: a
// depthwise causal conv over the mixed QKV channels whose inputs are cached
// for decode).  Per sequence b, channel c, token t:
//     y[b,t,c] = act(bias[c] + sum_{j<K} w[c][j] x[b, t-K+1+j, c]),
// inputs before token 0 from the cached state [B][K-1][C] (or zero).
// A streaming kernel (about a dozen flops per 4 bytes moved).  A work-group of
// eight waves covers 256 channels of 64 consecutive tokens: a thread owns 4
// channels (8-byte accesses for bfloat16, 16-byte for float32, non-temporal
// stores) of one wave's 8 tokens and keeps its window (its 8 rows plus the K-1
// rows before them) in registers, issuing all its row loads before any
// arithmetic.  Each wave hands its last K-1 rows to the next wave through LDS,
// so only the work-group's first wave loads a halo: the input is read 67/64
// times (with a halo per 16-token thread block it was 19/16, 1.10x the minimum
// traffic).  Four channels per thread keep a thread near 70 registers, so six
// waves share a SIMD and one wave's arithmetic overlaps the others' loads.  The new state (the last K-1 inputs) is written
// by the first wave of the first token block, which is also the only reader of
// the old state: in-place state update is race-free.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

constexpr int CONV_TT = 8;                       // tokens per thread (one wave's block)
constexpr int CONV_CH = 4;                       // channels per thread
constexpr int CONV_WAVES = 8;                    // consecutive token blocks per work-group
constexpr int CONV_BT = CONV_TT * CONV_WAVES;    // tokens per work-group
constexpr int CONV_BC = 64 * CONV_CH;            // channels per work-group

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
__global__ __launch_bounds__(64 * CONV_WAVES) void causal_conv1d_kernel(ConvArgs p) {
    typedef Row4<E> R4;
    typedef typename R4::raw raw;
    constexpr int W = CONV_TT + K - 1;  // rows in the window
    // bfloat16 SiLU with log2 e folded into the weights and bias: a = x log2 e
    // and x sigmoid(x) = a / (log2 e (1 + 2^-a)), one exp2, one fma, one
    // reciprocal, one multiply.  float32 keeps the exact-exponential sigmoid.
    constexpr bool FOLD = SILU && sizeof(E) == 2;
    constexpr float L2E = 1.4426950408889634f, WS = FOLD ? L2E : 1.f;
    __shared__ raw hand[CONV_WAVES - 1][K - 1][64];  // wave w's last K-1 rows, for wave w + 1

    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c0 = blockIdx.x * CONV_BC + lane * CONV_CH;
    const bool valid = c0 < p.C;  // no early exit: every thread reaches the barrier
    const int b = blockIdx.z, T = p.T, C = p.C;
    const int t0 = blockIdx.y * CONV_BT + wv * CONV_TT;  // this wave's first token
    const void *state = p.state;

    // own rows t0 .. t0+15 into win[K-1 ..]: full blocks take straight-line
    // loads from one base offset (a per-row bound test put scalar branches in
    // front of every load and cut the bytes in flight)
    raw win[W];
#pragma unroll
    for (int i = 0; i < W; ++i) win[i] = R4::zero();
    if (valid) {
        const size_t base = ((size_t)b * T + t0) * C + c0;
        if (t0 + CONV_TT <= T) {
#pragma unroll
            for (int i = 0; i < CONV_TT; ++i) win[K - 1 + i] = R4::ld(p.x, base + (size_t)i * C);
        } else {
#pragma unroll
            for (int i = 0; i < CONV_TT; ++i)
                if (t0 + i < T) win[K - 1 + i] = R4::ld(p.x, base + (size_t)i * C);
        }
        if (wv == 0) {  // the work-group's halo: earlier inputs, the cached state, or zeros
#pragma unroll
            for (int i = 0; i < K - 1; ++i) {
                const int s = t0 - (K - 1) + i;
                if (s >= 0 && s < T) win[i] = R4::ld(p.x, ((size_t)b * T + s) * C + c0);
                else if (s < 0 && state) win[i] = R4::ld(state, ((size_t)b * (K - 1) + (K - 1 + s)) * C + c0);
            }
        }
    }
    // weights and bias after the window, with no branch around a load: a
    // guarded load's wait would also wait for every window row issued before it
    const int cw = valid ? c0 : 0;
    const f4 *wp = reinterpret_cast<const f4 *>(p.w + (size_t)cw * K);
    const float *bp = p.bias ? p.bias : p.w;  // any valid address when there is no bias
    const bool has_bias = p.bias != nullptr;
    float w[CONV_CH][K], bias[CONV_CH];
#pragma unroll
    for (int j = 0; j < CONV_CH; ++j) {
        static_assert(K == 4, "one float4 of weights per channel");
        const f4 wj = wp[j];
#pragma unroll
        for (int k = 0; k < K; ++k) w[j][k] = wj[k] * WS;
        const float bj = bp[cw + j];
        bias[j] = has_bias ? bj * WS : 0.f;
    }
    // hand-over: the last K-1 own rows go to the next wave, whose halo they are
    if (wv < CONV_WAVES - 1) {
#pragma unroll
        for (int i = 0; i < K - 1; ++i) hand[wv][i][lane] = win[CONV_TT + i];
    }
    __syncthreads();
    if (wv > 0) {
#pragma unroll
        for (int i = 0; i < K - 1; ++i) win[i] = hand[wv - 1][i][lane];
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
    const int nout = valid ? (T - t0 < CONV_TT ? T - t0 : CONV_TT) : 0;  // outputs of this thread
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
    if (blockIdx.y == 0 && wv == 0 && valid && p.state_out) {
        // the last K-1 inputs; older cached inputs when T < K-1
#pragma unroll
        for (int i = 0; i < K - 1; ++i) {
            const int s = T - (K - 1) + i;
            raw r = R4::zero();
            if (s >= 0) r = R4::ld(p.x, ((size_t)b * T + s) * C + c0);
            // cached slot K-1+s = T+i >= i: not yet overwritten when the state is updated in place
            else if (state) r = R4::ld(state, ((size_t)b * (K - 1) + (K - 1 + s)) * C + c0);
            R4::st(p.state_out, ((size_t)b * (K - 1) + i) * C + c0, r);
        }
    }
}

template <typename T, bool SILU>
static hipError_t launch_conv_t(const ConvArgs &p, hipStream_t s) {
    const dim3 grid((unsigned)((p.C + CONV_BC - 1) / CONV_BC),
                    (unsigned)(p.T > 0 ? (p.T + CONV_BT - 1) / CONV_BT : 1), (unsigned)p.B);
    hipLaunchKernelGGL((causal_conv1d_kernel<T, 4, SILU>), grid, dim3(64 * CONV_WAVES), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_causal_conv1d(const ConvArgs &p, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    if (p.K != 4 || p.C % CONV_CH || p.qk % CONV_CH) return hipErrorInvalidValue;
    if (p.f32) return p.silu ? launch_conv_t<float, true>(p, s) : launch_conv_t<float, false>(p, s);
    return p.silu ? launch_conv_t<bf16_t, true>(p, s) : launch_conv_t<bf16_t, false>(p, s);
}

int conv_tokens_per_block() { return CONV_BT; }

}  // namespace gdn
