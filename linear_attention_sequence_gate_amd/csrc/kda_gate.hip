// KDA gate kernel and the optional decay-range check.
//
// Gate ("Kimi K3 internal structure analysis", section "Sequence mixing: 3 KDA
// layers per global MLA layer"): g = -5 * sigmoid(exp(A[h,c]) * z[b,t,h,c]).
// Purely elementwise and HBM-bound: it reads z (2 or 4 B) and writes g (4 B)
// per element, so each thread moves 8 elements with 16/32-byte vector
// accesses and exp(A) is recomputed from the small, L2-resident A table.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// Eight consecutive inputs as fp32 (16-byte loads; bases are 16-byte aligned).
__device__ __forceinline__ void load8(const bf16 *p, float *out) {
    bf16x8 v = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(p));
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = (float)v[j];
}
__device__ __forceinline__ void load8(const float *p, float *out) {
    floatx4 a = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(p));
    floatx4 b = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(p) + 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) { out[j] = a[j]; out[4 + j] = b[j]; }
}

template <typename T>
__global__ __launch_bounds__(256) void gate_kernel(const T *__restrict__ z,
                                                   const float *__restrict__ A,
                                                   float *__restrict__ g, int64_t n8,
                                                   int HD) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
        float zv[8];
        load8(z + i * 8, zv);
        // 8 consecutive elements share the head and sit at channels c..c+7 of
        // the [H, dk] table (dk is a multiple of 8).
        const float *a = A + (int)((i * 8) % HD);
        float out[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            out[j] = gate_value(a[j], zv[j]);
        floatx4 *gp = reinterpret_cast<floatx4 *>(g + i * 8);
        __builtin_nontemporal_store(floatx4{out[0], out[1], out[2], out[3]}, gp);
        __builtin_nontemporal_store(floatx4{out[4], out[5], out[6], out[7]}, gp + 1);
    }
}

// Counts elements with g outside [-5, 0] and aligned 16-token tiles whose
// fp32 running sum drops below -80.  One thread per (b, tile, h, c).
__global__ __launch_bounds__(256) void range_check_kernel(const float *__restrict__ g,
                                                          int64_t B, int64_t T, int64_t H,
                                                          int64_t dk,
                                                          unsigned int *__restrict__ bad) {
    const int64_t ntile = (T + kSub - 1) / kSub;
    const int64_t total = B * ntile * H * dk;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t c = i % dk;
        const int64_t h = (i / dk) % H;
        const int64_t tile = (i / (dk * H)) % ntile;
        const int64_t b = i / (dk * H * ntile);
        float sum = 0.0f;
        unsigned int nbad = 0;
        for (int r = 0; r < kSub; ++r) {
            const int64_t t = tile * kSub + r;
            if (t >= T) break;
            const float x = g[((b * T + t) * H + h) * dk + c];
            if (!(x >= kGmin && x <= 0.0f)) ++nbad;   // also catches NaN
            sum += x;
        }
        if (!(sum >= kGmin * kSub)) ++nbad;
        if (nbad) atomicAdd(bad, nbad);
    }
}

static int grid_for(int64_t work, int block) {
    int64_t blocks = (work + block - 1) / block;
    const int64_t cap = 256 * 64;   // enough to fill 256 CUs many times over
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    return (int)blocks;
}

hipError_t launch_gate(const void *z, const float *A, float *g, int64_t n_elems, int H, int dk,
                       int is_bf16, hipStream_t s) {
    const int64_t n8 = n_elems / 8;
    const int grid = grid_for(n8, 256);
    if (is_bf16)
        hipLaunchKernelGGL(gate_kernel<bf16>, dim3(grid), dim3(256), 0, s,
                           static_cast<const bf16 *>(z), A, g, n8, H * dk);
    else
        hipLaunchKernelGGL(gate_kernel<float>, dim3(grid), dim3(256), 0, s,
                           static_cast<const float *>(z), A, g, n8, H * dk);
    return hipGetLastError();
}

hipError_t launch_range_check(const float *g, int64_t B, int64_t T, int64_t H, int64_t dk,
                              unsigned int *bad, hipStream_t s) {
    const int64_t ntile = (T + kSub - 1) / kSub;
    const int grid = grid_for(B * ntile * H * dk, 256);
    hipLaunchKernelGGL(range_check_kernel, dim3(grid), dim3(256), 0, s, g, B, T, H, dk, bad);
    return hipGetLastError();
}

}  // namespace kda
