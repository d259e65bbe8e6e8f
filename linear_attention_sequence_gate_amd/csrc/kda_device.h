// Device-side helpers shared by the KDA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Gate floor: g = kGmin * sigmoid(exp(A) * z)  ("Kimi K3 internal structure
// analysis", section "Sequence mixing: 3 KDA layers per global MLA layer").
constexpr float kGmin = -5.0f;
// Chunk length and the subtile length whose cumulative log-decay the floor
// bounds by 16 * 5 = 80 (same section).
constexpr int kChunk = 64;
constexpr int kSub = 16;

typedef __bf16 bf16;
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// element conversion (bf16 <-> fp32 uses round-to-nearest-even)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

// Four fp32 -> bf16 (round to nearest even).
__device__ __forceinline__ bf16x4 to_bf16x4(floatx4 x) {
    // pairwise, so each pair maps onto one packed conversion
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const bf16x2 a = __builtin_convertvector(floatx2{x[0], x[1]}, bf16x2);
    const bf16x2 b = __builtin_convertvector(floatx2{x[2], x[3]}, bf16x2);
    return __builtin_bit_cast(bf16x4, u32x2{__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b)});
}

// x = hi + lo to about 2^-17 relative: hi = bf16(x), lo = bf16(x - hi).  hi
// is widened back to fp32 from its packed bits (two bf16 per dword) instead
// of being converted a second time.
__device__ __forceinline__ void split_bf16(floatx4 x, bf16x4 &hi, bf16x4 &lo) {
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    hi = __builtin_convertvector(x, bf16x4);
    const u32x2 w = __builtin_bit_cast(u32x2, hi);
    const floatx4 hf = {__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                        __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
    lo = __builtin_convertvector(x - hf, bf16x4);
}

// Store four consecutive values (8 B for bf16, 16 B for fp32); p must be aligned.
__device__ __forceinline__ void store4(float *p, float a, float b, float c, float d) {
    *reinterpret_cast<floatx4 *>(p) = floatx4{a, b, c, d};
}
__device__ __forceinline__ void store4(bf16 *p, float a, float b, float c, float d) {
    *reinterpret_cast<bf16x4 *>(p) = to_bf16x4(floatx4{a, b, c, d});
}

// ---------------------------------------------------------------------------
// The gate, one element: g = -5 * sigmoid(exp(a) * z), evaluated so that no
// exponential overflows.  Used by the gate kernel and the fused decode step,
// so the gate has a single device definition.
// ---------------------------------------------------------------------------
// ea = exp(a): kernels that reuse one channel's exp(a) take it once
__device__ __forceinline__ float gate_value_ea(float ea, float z) {
    float x = ea * z;
    float e = expf(-fabsf(x));              // in (0, 1]
    float s = (x >= 0.0f) ? 1.0f / (1.0f + e) : e / (1.0f + e);
    return kGmin * s;
}
__device__ __forceinline__ float gate_value(float a, float z) { return gate_value_ea(expf(a), z); }

// The same gate for kernels that evaluate it inline on every element, with
// the hardware's base-2 exponential and reciprocal and the per-channel part
// taken once: with zc = -log2(e) e^{a},
//     sigmoid(e^{a} z) = 1 / (1 + 2^{zc z}),   log2(alpha) = -5 log2(e) sigmoid(e^{a} z).
// A very negative argument overflows 2^{zc z} to +inf and the reciprocal to
// 0, i.e. g = 0, its limit; a very positive one gives 2^{..} = 0 and g = -5.
// Each step is within a few ulp of gate_value.
__device__ __forceinline__ floatx2 gate_zscale2(const float *a) {
    constexpr float kNegLog2e = -1.4426950408889634f;
    return floatx2{kNegLog2e * expf(a[0]), kNegLog2e * expf(a[1])};
}
__device__ __forceinline__ floatx2 gate_log2_alpha2(floatx2 zc, floatx2 z) {
    constexpr float kGminLog2e = kGmin * 1.4426950408889634f;
    floatx2 r;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const float t = __builtin_amdgcn_exp2f(zc[j] * z[j]);
        r[j] = kGminLog2e * __builtin_amdgcn_rcpf(1.0f + t);
    }
    return r;
}

// ---------------------------------------------------------------------------
// 16x16 MFMA tile products in "both operands k-contiguous" form:
//   out[m][n] += sum_k X[m][k] * Y[n][k]
// X and Y live in LDS with row pitches ldx, ldy (elements).  After the call,
// lane l holds out[4*(l/16) + j][l % 16] in acc[j], j = 0..3 (the standard
// 16x16 accumulator layout).  Each lane feeds the same k positions of X and Y
// into the same operand slots, so the hardware's k ordering inside one
// instruction does not matter.
// ---------------------------------------------------------------------------
template <typename T> struct Mma;

template <> struct Mma<bf16> {
    static constexpr int kStep = 32;            // k per instruction
    __device__ __forceinline__ static void step(floatx4 &acc, const bf16 *x, const bf16 *y) {
        bf16x8 a = *reinterpret_cast<const bf16x8 *>(x);
        bf16x8 b = *reinterpret_cast<const bf16x8 *>(y);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
};

template <> struct Mma<float> {
    static constexpr int kStep = 16;            // four 16x16x4 instructions
    __device__ __forceinline__ static void step(floatx4 &acc, const float *x, const float *y) {
        floatx4 a = *reinterpret_cast<const floatx4 *>(x);
        floatx4 b = *reinterpret_cast<const floatx4 *>(y);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
    }
};

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations
// and meets the other waves, but leaves global loads in flight (a plain
// __syncthreads also drains them, which would expose the latency of loads
// prefetched for a later stage).  No global memory is exchanged between the
// threads of a workgroup in these kernels.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// K must be a multiple of Mma<T>::kStep.
template <typename T>
__device__ __forceinline__ void tile_mma(floatx4 &acc, const T *X, int ldx, const T *Y, int ldy,
                                         int K, int lane) {
    constexpr int kq = Mma<T>::kStep / 4;       // k elements per lane per step
    const int r = lane & 15, grp = lane >> 4;
    const T *xp = X + r * ldx + grp * kq;
    const T *yp = Y + r * ldy + grp * kq;
    for (int k0 = 0; k0 < K; k0 += Mma<T>::kStep)
        Mma<T>::step(acc, xp + k0, yp + k0);
}

}  // namespace kda
