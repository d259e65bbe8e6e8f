// KDA single-token decode step with the gate fused, state updated in place.
//
// Per (sequence n, head h), with alpha = exp(g), g = -5 sigmoid(exp(A) z):
//     r1 = (Diag(alpha) S)^T k,   r2 = (Diag(alpha) S)^T q,   kappa = k . q
//     u  = beta (v - r1),         o  = r2 + kappa u
//     S  <- Diag(alpha) S + k u^T
// which is the recurrence of "Kimi K3 internal structure analysis" (section
// "Sequence mixing: 3 KDA layers per global MLA layer": retention applied
// before the delta-rule write) for one token, rewritten so the state is read
// once and written once: o = S_new^T q = (alpha S)^T q + (k . q) u.
//
// The step is HBM-bound (64 KiB read + 64 KiB written per head at d = 128 for
// ~115 kflop), so the design goal is a single coalesced sweep: one 256-thread
// workgroup per head, each thread holding a float4 column group of
// DK / (256 / (DV/4)) rows in registers between the reduction and the write.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

template <typename T>
__device__ __forceinline__ float ld1(const T *p) { return to_f32(*p); }

template <typename T, int DK, int DV>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ z, const float *__restrict__ A, const T *__restrict__ beta,
    float *__restrict__ state, T *__restrict__ o, int H) {
    constexpr int NCG = DV / 4;          // float4 column groups
    constexpr int RG = 256 / NCG;        // row groups
    constexpr int ROWS = DK / RG;        // rows per thread
    static_assert(ROWS >= 1 && DK % RG == 0, "shape");
    constexpr int GPW = 64 / NCG;        // row groups inside one wave

    __shared__ float sAlpha[DK], sK[DK], sQ[DK];
    __shared__ float sV[DV];
    __shared__ floatx4 sRed[4][2][NCG];
    __shared__ float sKq[4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = tid % NCG, rg = tid / NCG;
    const int64_t nh = blockIdx.x;
    const int h = (int)(nh % H);

    // 1. issue the state loads first: they are the bulk of the traffic
    floatx4 *Sp = reinterpret_cast<floatx4 *>(state + nh * (int64_t)(DK * DV));
    floatx4 s[ROWS];
#pragma unroll
    for (int i = 0; i < ROWS; ++i) s[i] = Sp[(rg + RG * i) * NCG + cg];

    // 2. per-channel gate, key and query, and the partial k . q
    float kq = 0.0f;
    if (tid < DK) {
        const int64_t off = nh * DK + tid;
        const float kk = ld1(k + off), qq = ld1(q + off);
        sAlpha[tid] = expf(gate_value(A[h * DK + tid], ld1(z + off)));
        sK[tid] = kk;
        sQ[tid] = qq;
        kq = kk * qq;
    }
    if (tid < DV) sV[tid] = ld1(v + nh * DV + tid);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) kq += __shfl_xor(kq, m);
    if (lane == 0) sKq[wave] = kq;
    __syncthreads();

    // 3. decay the rows and accumulate the two projections
    floatx4 r1 = {0, 0, 0, 0}, r2 = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int c = rg + RG * i;
        const float a = sAlpha[c];
        s[i] *= a;
        r1 += s[i] * sK[c];
        r2 += s[i] * sQ[c];
    }
    // reduce over the row groups: first inside the wave ...
#pragma unroll
    for (int m = NCG; m < 64; m <<= 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            r1[j] += __shfl_xor(r1[j], m);
            r2[j] += __shfl_xor(r2[j], m);
        }
    }
    // ... then across the four waves
    if (lane < NCG) {
        sRed[wave][0][cg] = r1;
        sRed[wave][1][cg] = r2;
    }
    __syncthreads();
    r1 = sRed[0][0][cg] + sRed[1][0][cg] + sRed[2][0][cg] + sRed[3][0][cg];
    r2 = sRed[0][1][cg] + sRed[1][1][cg] + sRed[2][1][cg] + sRed[3][1][cg];
    const float kappa = sKq[0] + sKq[1] + sKq[2] + sKq[3];
    const float bt = ld1(beta + nh);

    floatx4 u;
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = bt * (sV[4 * cg + j] - r1[j]);

    // 4. write the new state in place and the output
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int c = rg + RG * i;
        Sp[c * NCG + cg] = s[i] + sK[c] * u;
    }
    if (rg == 0) {
        floatx4 ov = r2 + kappa * u;
        store4(o + nh * DV + 4 * cg, ov[0], ov[1], ov[2], ov[3]);
    }
    (void)GPW;
}

template <typename T, int DK>
static hipError_t decode_dv(const void *q, const void *k, const void *v, const void *z,
                            const float *A, const void *beta, float *state, void *o,
                            int64_t NH, int H, int dv, hipStream_t s) {
#define KDA_DECODE(DV)                                                                      \
    hipLaunchKernelGGL((decode_step_kernel<T, DK, DV>), dim3((unsigned)NH), dim3(256), 0, s, \
                       (const T *)q, (const T *)k, (const T *)v, (const T *)z, A,           \
                       (const T *)beta, state, (T *)o, H)
    switch (dv) {
    case 32: KDA_DECODE(32); break;
    case 64: KDA_DECODE(64); break;
    case 128: KDA_DECODE(128); break;
    default: return hipErrorInvalidValue;
    }
#undef KDA_DECODE
    return hipGetLastError();
}

template <typename T>
static hipError_t decode_dk(const void *q, const void *k, const void *v, const void *z,
                            const float *A, const void *beta, float *state, void *o,
                            int64_t NH, int H, int dk, int dv, hipStream_t s) {
    switch (dk) {
    case 32: return decode_dv<T, 32>(q, k, v, z, A, beta, state, o, NH, H, dv, s);
    case 64: return decode_dv<T, 64>(q, k, v, z, A, beta, state, o, NH, H, dv, s);
    case 128: return decode_dv<T, 128>(q, k, v, z, A, beta, state, o, NH, H, dv, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_step(const void *q, const void *k, const void *v, const void *z,
                              const float *A, const void *beta, float *state, void *o,
                              int64_t N, int64_t H, int dk, int dv, int is_bf16, hipStream_t s) {
    const int64_t NH = N * H;
    if (is_bf16)
        return decode_dk<bf16>(q, k, v, z, A, beta, state, o, NH, (int)H, dk, dv, s);
    return decode_dk<float>(q, k, v, z, A, beta, state, o, NH, (int)H, dk, dv, s);
}

}  // namespace kda
