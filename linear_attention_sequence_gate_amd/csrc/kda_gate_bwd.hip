// Reverse mode of the KDA gate ("Kimi K3 internal structure analysis",
// section "Sequence mixing: 3 KDA layers per global MLA layer": g = -5 *
// sigmoid(exp(A[h,c]) * z[b,t,h,c])).  The pages say nothing of training; with
// x = exp(A) z and L = <g, dg>:
//     dz = -5 sigmoid'(x) exp(A) dg
//     dA = sum over rows (b, t) of -5 sigmoid'(x) x dg
// where sigmoid'(x) = e^{-|x|} / (1 + e^{-|x|})^2, the form that stays exact
// for large |x| (no 1 - sigmoid cancellation).
//
// HBM-bound: it reads z and dg and writes dz once.  A thread owns one column
// (h, c) over a range of rows, so every access of a wave is one contiguous
// span, and keeps its column's share of dA in a register; the shares of the
// row ranges are added in a fixed order by a second small kernel, so dA does
// not depend on scheduling.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kGbCols = 256;                     // columns per workgroup

// Row ranges (dA shares per column): about 1024 workgroups in all, at most 256.
int gate_bwd_splits(int64_t rows, int C) {
    const int tiles = (C + kGbCols - 1) / kGbCols;
    int64_t s = 1024 / tiles;
    if (s < 1) s = 1;
    if (s > 256) s = 256;
    if (s > rows) s = rows;
    return (int)s;
}

template <typename T>
__global__ __launch_bounds__(kGbCols) void gate_bwd_kernel(const T *__restrict__ z,
                                                           const float *__restrict__ A,
                                                           const float *__restrict__ dg,
                                                           float *__restrict__ dz,
                                                           float *__restrict__ part, int64_t rows,
                                                           int C, int64_t rows_per_split) {
    const int col = blockIdx.x * kGbCols + threadIdx.x;
    if (col >= C) return;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_split;
    const int64_t r1 = r0 + rows_per_split < rows ? r0 + rows_per_split : rows;
    const float eA = expf(A[col]);
    float acc = 0.f;
#pragma unroll 4
    for (int64_t r = r0; r < r1; ++r) {
        const int64_t i = r * C + col;
        const float x = eA * to_f32(z[i]);
        const float e = expf(-fabsf(x));
        const float d = 1.f + e;
        const float t = kGmin * dg[i] * e / (d * d);
        dz[i] = t * eA;
        acc += t * x;
    }
    part[(int64_t)blockIdx.y * C + col] = acc;
}

__global__ __launch_bounds__(kGbCols) void gate_bwd_sum_kernel(const float *__restrict__ part,
                                                               float *__restrict__ dA, int splits,
                                                               int C) {
    const int col = blockIdx.x * kGbCols + threadIdx.x;
    if (col >= C) return;
    float s = 0.f;
#pragma unroll 8
    for (int k = 0; k < splits; ++k) s += part[(int64_t)k * C + col];
    dA[col] = s;
}

size_t gate_bwd_workspace_bytes(int64_t rows, int C) {
    return (size_t)gate_bwd_splits(rows, C) * (size_t)C * sizeof(float);
}

hipError_t launch_gate_bwd(const void *z, const float *A, const float *dg, float *dz, float *dA,
                           float *part, int64_t rows, int H, int dk, int is_bf16, hipStream_t s) {
    const int C = H * dk;
    const int splits = gate_bwd_splits(rows, C);
    const int64_t rps = (rows + splits - 1) / splits;
    const dim3 grid((unsigned)((C + kGbCols - 1) / kGbCols), (unsigned)splits);
    if (is_bf16)
        hipLaunchKernelGGL(gate_bwd_kernel<bf16>, grid, dim3(kGbCols), 0, s,
                           static_cast<const bf16 *>(z), A, dg, dz, part, rows, C, rps);
    else
        hipLaunchKernelGGL(gate_bwd_kernel<float>, grid, dim3(kGbCols), 0, s,
                           static_cast<const float *>(z), A, dg, dz, part, rows, C, rps);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gate_bwd_sum_kernel, dim3((unsigned)((C + kGbCols - 1) / kGbCols)),
                       dim3(kGbCols), 0, s, part, dA, splits, C);
    return hipGetLastError();
}

}  // namespace kda
