// gdn_device.h -- device-side helpers for the gfx950 Gated DeltaNet kernels:
// vector types, bfloat16/float16 conversions, gate functions and MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

// bfloat16 is carried as its 16-bit pattern.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}

// float32 -> bfloat16, round-to-nearest-even, NaN kept a NaN: the hardware
// converter (v_cvt_pk_bf16_f32 on gfx950; a software rounding with a NaN test
// cost several instructions and a branch per element)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Ordering of LDS accesses among the lanes of one wave (no work-group barrier):
// complete this wave's outstanding LDS operations and keep the compiler from
// moving LDS accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Inclusive prefix sum of a double over the 64 lanes of a wave, by DPP moves
// of its two 32-bit halves (no LDS): shifts by 1, 2, 4, 8 inside each row of
// 16 lanes, then lane 15 of each row into the next row and lane 31 into rows
// 2 and 3.  Disabled or out-of-row sources read 0 (= +0.0).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double v) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)b, CTRL, ROW_MASK, 0xf, true);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, ROW_MASK, 0xf, true);
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ double wave_prefix_sum_f64(double x) {
    x += dpp_f64<0x111, 0xf>(x);  // row_shr:1
    x += dpp_f64<0x112, 0xf>(x);  // row_shr:2
    x += dpp_f64<0x114, 0xf>(x);  // row_shr:4
    x += dpp_f64<0x118, 0xf>(x);  // row_shr:8
    x += dpp_f64<0x142, 0xa>(x);  // row_bcast:15 into rows 1, 3
    x += dpp_f64<0x143, 0xc>(x);  // row_bcast:31 into rows 2, 3
    return x;
}

// Element-type traits of q/k/v/out.
template <typename T> struct io;
template <> struct io<float> {
    __device__ static __forceinline__ float ld(const float *p, size_t i) { return p[i]; }
    __device__ static __forceinline__ void st(float *p, size_t i, float x) { p[i] = x; }
};
template <> struct io<bf16_t> {
    __device__ static __forceinline__ float ld(const bf16_t *p, size_t i) {
        return bf16_to_f32(reinterpret_cast<const uint16_t *>(p)[i]);
    }
    __device__ static __forceinline__ void st(bf16_t *p, size_t i, float x) {
        reinterpret_cast<uint16_t *>(p)[i] = f32_to_bf16(x);
    }
};

// Load 4 consecutive elements as float4 (p + i must be 8-byte aligned for
// bf16, 16-byte aligned for float).
__device__ __forceinline__ f4 ld4(const float *p, size_t i) {
    return *reinterpret_cast<const f4 *>(p + i);
}
__device__ __forceinline__ f4 ld4(const bf16_t *p, size_t i) {
    u16x4 u = *reinterpret_cast<const u16x4 *>(reinterpret_cast<const uint16_t *>(p) + i);
    return f4{bf16_to_f32(u[0]), bf16_to_f32(u[1]), bf16_to_f32(u[2]), bf16_to_f32(u[3])};
}
// Load 8 consecutive elements as two float4 (16-byte aligned for bf16,
// 32-byte aligned pair of float4 for float).
__device__ __forceinline__ void ld8(const float *p, size_t i, f4 &lo, f4 &hi) {
    lo = *reinterpret_cast<const f4 *>(p + i);
    hi = *reinterpret_cast<const f4 *>(p + i + 4);
}
__device__ __forceinline__ void ld8(const bf16_t *p, size_t i, f4 &lo, f4 &hi) {
    u16x8 u = *reinterpret_cast<const u16x8 *>(reinterpret_cast<const uint16_t *>(p) + i);
    lo = f4{bf16_to_f32(u[0]), bf16_to_f32(u[1]), bf16_to_f32(u[2]), bf16_to_f32(u[3])};
    hi = f4{bf16_to_f32(u[4]), bf16_to_f32(u[5]), bf16_to_f32(u[6]), bf16_to_f32(u[7])};
}
__device__ __forceinline__ void st4(float *p, size_t i, f4 x) {
    *reinterpret_cast<f4 *>(p + i) = x;
}
__device__ __forceinline__ void st4(bf16_t *p, size_t i, f4 x) {
    u16x4 u = {f32_to_bf16(x[0]), f32_to_bf16(x[1]), f32_to_bf16(x[2]), f32_to_bf16(x[3])};
    *reinterpret_cast<u16x4 *>(reinterpret_cast<uint16_t *>(p) + i) = u;
}

// Gate functions in float32 (dingfen page, sections 9-10).
// softplus(x) = log(1 + e^x), evaluated as x + log(1 + e^-x) for x > 0.
__device__ __forceinline__ float softplus_f32(float x) {
    return x > 0.f ? x + log1pf(expf(-x)) : log1pf(expf(x));
}
__device__ __forceinline__ float sigmoid_f32(float x) { return 1.f / (1.f + expf(-x)); }
// The same gates from the hardware base-2 exponential and logarithm and the
// hardware reciprocal (a few ulp): used where the operands are float16 and the
// output bfloat16, whose rounding is orders of magnitude coarser.  softplus
// keeps its absolute error near float32 rounding: max(x, 0) + log(1 + e^-|x|).
__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ __forceinline__ float softplus_fast(float x) {
    return fmaxf(x, 0.f) + __builtin_amdgcn_logf(1.f + exp_fast(-fabsf(x))) * 0.6931471805599453f;
}
__device__ __forceinline__ float sigmoid_fast(float x) { return __builtin_amdgcn_rcpf(1.f + exp_fast(-x)); }

// ---------------------------------------------------------------------------
// MFMA on 16x16 output tiles.  Layouts (checked on gfx950):
//   accumulator: lane l holds C[4*(l/16) + i][l%16], i = 0..3
//   16x16x32 f16: lane l holds A[l%16][8*(l/16) + j], B[8*(l/16) + j][l%16], j = 0..7
//   16x16x4  f32: lane l holds A[l%16][l/16],        B[l/16][l%16]
// Any permutation of the contraction index that A and B share gives the same
// product; the kernels use "k-block" operands: for a 16-deep block of the
// contraction, lane l supplies the 4 values with k = 4*(l/16) + i, i = 0..3 --
// exactly the rows an accumulator tile holds, so an accumulator tile can feed
// the next product as its B operand without any data movement.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f4 mfma_f16_k32(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma_f16_k16(h4 a, h4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma_f32_k4(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ h4 to_h4(f4 x) { return __builtin_convertvector(x, h4); }
__device__ __forceinline__ h8 cat_h8(h4 a, h4 b) {
    return h8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Operand element type of the matrix-core products: float16 for bf16 inputs,
// float32 for float32 inputs.
template <bool F32> struct mma;

template <> struct mma<false> {
    typedef _Float16 E;
    typedef h4 V4;  // one k-block operand (4 values per lane)
    __device__ static __forceinline__ V4 from_f4(f4 x) { return to_h4(x); }
    // acc += A(block) * B(block): one 16-deep k-block
    __device__ static __forceinline__ f4 block(f4 acc, V4 a, V4 b) { return mfma_f16_k16(a, b, acc); }
    // acc += A(blocks kb0,kb1) * B(blocks kb0,kb1): two 16-deep k-blocks per instruction
    __device__ static __forceinline__ f4 pair(f4 acc, V4 a0, V4 a1, V4 b0, V4 b1) {
        return mfma_f16_k32(cat_h8(a0, a1), cat_h8(b0, b1), acc);
    }
};

template <> struct mma<true> {
    typedef float E;
    typedef f4 V4;
    __device__ static __forceinline__ V4 from_f4(f4 x) { return x; }
    __device__ static __forceinline__ f4 block(f4 acc, V4 a, V4 b) {
        acc = mfma_f32_k4(a[0], b[0], acc);
        acc = mfma_f32_k4(a[1], b[1], acc);
        acc = mfma_f32_k4(a[2], b[2], acc);
        acc = mfma_f32_k4(a[3], b[3], acc);
        return acc;
    }
    __device__ static __forceinline__ f4 pair(f4 acc, V4 a0, V4 a1, V4 b0, V4 b1) {
        acc = block(acc, a0, b0);
        return block(acc, a1, b1);
    }
};

}  // namespace gdn
