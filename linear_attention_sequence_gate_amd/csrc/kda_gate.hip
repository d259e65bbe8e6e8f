// KDA gate kernel and the optional decay-range check.
//
// Gate ("Kimi K3 internal structure analysis", section "Sequence mixing: 3 KDA
// layers per global MLA layer"): g = -5 * sigmoid(exp(A[h,c]) * z[b,t,h,c]).
// Purely elementwise and HBM-bound: it reads z (2 or 4 B) and writes g (4 B)
// per element with coalesced vector accesses; exp(A) is recomputed from the
// small, L2-resident A table.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// Four consecutive inputs as fp32 (8- or 16-byte loads; bases are aligned).
__device__ __forceinline__ floatx4 load4(const bf16 *p) {
    const bf16x4 v = __builtin_nontemporal_load(reinterpret_cast<const bf16x4 *>(p));
    return floatx4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ floatx4 load4(const float *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(p));
}

// Element groups of four: a wave handles 128 consecutive groups per pass, lane
// l groups l and l + 64, so every load and store instruction of the wave
// covers one contiguous span (partial cache-line writes would cost extra
// HBM traffic).  The [H, dk] table index of a group is kept incrementally.
template <typename T>
__global__ __launch_bounds__(256) void gate_kernel(const T *__restrict__ z,
                                                   const float *__restrict__ A,
                                                   float *__restrict__ g, int64_t n4, int HD4) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t step = (((int64_t)gridDim.x * blockDim.x) >> 6) * 128;
    const int dstep = (int)(step % HD4);
    int64_t q = wave * 128 + lane;
    int c0 = (int)(q % HD4), c1 = (int)((q + 64) % HD4);
    // exp(A) of this lane's two groups; the groups keep their channels from
    // one pass to the next when the stride is a multiple of H dk (dstep = 0,
    // the usual case), so it is evaluated again only when they move
    auto expA = [&](int c) {
        const floatx4 a = *reinterpret_cast<const floatx4 *>(A + 4 * c);
        return floatx4{expf(a[0]), expf(a[1]), expf(a[2]), expf(a[3])};
    };
    floatx4 ea0 = expA(c0), ea1 = expA(c1);
    // UNR passes per loop trip when the groups keep their channels: every
    // pass's loads are issued before any pass is computed, so each thread
    // keeps 2 UNR loads in flight
    constexpr int UNR = 2;
    if (dstep == 0) {
        for (; q + (UNR - 1) * step + 64 < n4; q += UNR * step) {
            floatx4 z0[UNR], z1[UNR];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                z0[u] = load4(z + 4 * (q + u * step));
                z1[u] = load4(z + 4 * (q + u * step + 64));
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                floatx4 g0, g1;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    g0[j] = gate_value_ea(ea0[j], z0[u][j]);
                    g1[j] = gate_value_ea(ea1[j], z1[u][j]);
                }
                __builtin_nontemporal_store(g0, reinterpret_cast<floatx4 *>(g + 4 * (q + u * step)));
                __builtin_nontemporal_store(g1, reinterpret_cast<floatx4 *>(g + 4 * (q + u * step + 64)));
            }
        }
    }
    for (; q < n4; q += step) {
        const bool two = q + 64 < n4;
        const floatx4 z0 = load4(z + 4 * q);
        const floatx4 z1 = two ? load4(z + 4 * (q + 64)) : floatx4{0, 0, 0, 0};
        floatx4 g0, g1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            g0[j] = gate_value_ea(ea0[j], z0[j]);
            g1[j] = gate_value_ea(ea1[j], z1[j]);
        }
        __builtin_nontemporal_store(g0, reinterpret_cast<floatx4 *>(g + 4 * q));
        if (two) __builtin_nontemporal_store(g1, reinterpret_cast<floatx4 *>(g + 4 * (q + 64)));
        if (dstep != 0) {
            c0 += dstep; if (c0 >= HD4) c0 -= HD4;
            c1 += dstep; if (c1 >= HD4) c1 -= HD4;
            ea0 = expA(c0);
            ea1 = expA(c1);
        }
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
    // n_elems and H * dk are multiples of dk, itself a multiple of 32
    const int64_t n4 = n_elems / 4;
    const int grid = grid_for((n4 + 1) / 2, 256);
    const int HD4 = H * dk / 4;
    if (is_bf16)
        hipLaunchKernelGGL(gate_kernel<bf16>, dim3(grid), dim3(256), 0, s,
                           static_cast<const bf16 *>(z), A, g, n4, HD4);
    else
        hipLaunchKernelGGL(gate_kernel<float>, dim3(grid), dim3(256), 0, s,
                           static_cast<const float *>(z), A, g, n4, HD4);
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
