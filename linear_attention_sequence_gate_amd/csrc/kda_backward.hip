// Reverse mode of the KDA recurrence, token by token.
//
// The forward step ("Kimi K3 internal structure analysis", section "Sequence
// mixing: 3 KDA layers per global MLA layer": retention before the delta-rule
// write; the read after it), for one (batch, head) chain and token t:
//     S' = Diag(a) S,  a = exp(g_t);   w = S'^T k;   u = beta (v - w)
//     S_t = S' + k u^T;                 o_t = S_t^T q
// and its reverse, given dS (the gradient with respect to S_t) and do_t:
//     dS += q do^T;            dq = S_t do
//     du = dS^T k;             dbeta = du . (v - w);   dv = beta du;   dw = -beta du
//     dk = dS u + S' dw;       dS' = dS + k dw^T
//     dg = a * rowsum(S * dS');  dS <- Diag(a) dS'
//
// One workgroup per chain holds S, the checkpoint it recomputes from, and dS
// in registers (a thread holds float4 column groups of ROWS rows, as in the
// decode kernel).  A first pass stores the state before every kCkpt-th token;
// the reverse pass walks the tokens backwards and recomputes the state before
// each token from its checkpoint (at most kCkpt - 1 forward steps).  Row sums
// (dk-vectors) reduce across the column lanes of a wave with lane exchanges;
// column sums (dv-vectors) across row groups through LDS.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kCkpt = 8;                         // tokens per checkpoint

template <int DK, int DV> struct BwdShape {
    static constexpr int TPB = DK * DV / 4 < 512 ? DK * DV / 4 : 512;
    static constexpr int NCG = DV / 4;           // float4 column groups
    static constexpr int RG = TPB / NCG;         // row groups
    static constexpr int ROWS = DK / RG;         // rows per thread
    static constexpr int NWV = TPB / 64;
    static_assert(ROWS >= 1 && DK % RG == 0 && TPB % 64 == 0 && NCG <= 64, "backward shape");
};

struct BwdArgs {
    const void *q, *k, *v, *beta, *dout;
    const float *g, *S0, *dST;
    float *ckpt;
    float *dq, *dk, *dv, *dg, *dbeta, *dS0;
    int64_t T;
    int H;
};

template <typename T> __device__ __forceinline__ float ldx(const void *p, int64_t i) {
    return to_f32(static_cast<const T *>(p)[i]);
}

// The token's inputs, broadcast through LDS.
template <int DK, int DV> struct BwdLds {
    float a[DK], k[DK], q[DK];
    float v[DV], dout[DV];
    float beta;
    floatx4 red[2][BwdShape<DK, DV>::NWV][BwdShape<DK, DV>::NCG];
};

template <typename T, int DK, int DV>
__device__ __forceinline__ void load_token(BwdLds<DK, DV> &L, const BwdArgs &a, int64_t row,
                                           bool with_read) {
    const int tid = threadIdx.x;
    if (tid < DK) {
        L.a[tid] = expf(a.g[row * DK + tid]);
        L.k[tid] = ldx<T>(a.k, row * DK + tid);
        if (with_read) L.q[tid] = ldx<T>(a.q, row * DK + tid);
    }
    if (tid < DV) {
        L.v[tid] = ldx<T>(a.v, row * DV + tid);
        if (with_read) L.dout[tid] = ldx<T>(a.dout, row * DV + tid);
    }
    if (tid == 0) L.beta = ldx<T>(a.beta, row);
}

// Sum over all rows of a per-thread float4 partial (one column group); the
// result is returned to every thread of that column group.  `buf` alternates
// so consecutive reductions need one barrier each.
template <int DK, int DV>
__device__ __forceinline__ floatx4 row_sum(BwdLds<DK, DV> &L, floatx4 x, int buf) {
    using Sh = BwdShape<DK, DV>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, cg = threadIdx.x % Sh::NCG;
#pragma unroll
    for (int m = Sh::NCG; m < 64; m <<= 1)
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] += __shfl_xor(x[j], m);
    if (lane < Sh::NCG) L.red[buf][wave][cg] = x;
    __syncthreads();
    floatx4 r = L.red[buf][0][cg];
#pragma unroll
    for (int w = 1; w < Sh::NWV; ++w) r += L.red[buf][w][cg];
    return r;
}

// Sum over the column groups (lanes of one row group); every lane of the
// group receives the total.
template <int NCG> __device__ __forceinline__ float col_sum(float x) {
#pragma unroll
    for (int m = 1; m < NCG; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

__device__ __forceinline__ float dot4(floatx4 x, floatx4 y) {
    return x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
}

// One forward step on the register state s (rows rg + RG i, column group cg).
template <typename T, int DK, int DV>
__device__ __forceinline__ void fwd_step(BwdLds<DK, DV> &L, const BwdArgs &a, int64_t row,
                                         floatx4 (&s)[BwdShape<DK, DV>::ROWS]) {
    using Sh = BwdShape<DK, DV>;
    const int cg = threadIdx.x % Sh::NCG, rg = threadIdx.x / Sh::NCG;
    load_token<T, DK, DV>(L, a, row, false);
    __syncthreads();
    floatx4 wp = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < Sh::ROWS; ++i) {
        const int c = rg + Sh::RG * i;
        s[i] *= L.a[c];
        wp += s[i] * L.k[c];
    }
    const floatx4 w = row_sum<DK, DV>(L, wp, 0);
    const floatx4 vv = {L.v[4 * cg], L.v[4 * cg + 1], L.v[4 * cg + 2], L.v[4 * cg + 3]};
    const floatx4 u = L.beta * (vv - w);
#pragma unroll
    for (int i = 0; i < Sh::ROWS; ++i) s[i] += L.k[rg + Sh::RG * i] * u;
    __syncthreads();                             // LDS inputs are rewritten next
}

template <typename T, int DK, int DV>
__global__ __launch_bounds__((BwdShape<DK, DV>::TPB)) void bwd_ckpt_kernel(BwdArgs a) {
    using Sh = BwdShape<DK, DV>;
    __shared__ BwdLds<DK, DV> L;
    const int bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
    const int cg = threadIdx.x % Sh::NCG, rg = threadIdx.x / Sh::NCG;
    const int64_t nck = (a.T + kCkpt - 1) / kCkpt;
    floatx4 s[Sh::ROWS];
#pragma unroll
    for (int i = 0; i < Sh::ROWS; ++i) {
        const int c = rg + Sh::RG * i;
        s[i] = a.S0 ? *reinterpret_cast<const floatx4 *>(a.S0 + ((int64_t)bh * DK + c) * DV + 4 * cg)
                    : floatx4{0, 0, 0, 0};
    }
    for (int64_t t = 0; t < a.T; ++t) {
        if (t % kCkpt == 0) {
            float *dst = a.ckpt + ((int64_t)bh * nck + t / kCkpt) * DK * DV;
#pragma unroll
            for (int i = 0; i < Sh::ROWS; ++i)
                *reinterpret_cast<floatx4 *>(dst + (rg + Sh::RG * i) * DV + 4 * cg) = s[i];
        }
        fwd_step<T, DK, DV>(L, a, ((int64_t)b * a.T + t) * a.H + h, s);
    }
}

template <typename T, int DK, int DV>
__global__ __launch_bounds__((BwdShape<DK, DV>::TPB)) void bwd_kernel(BwdArgs a) {
    using Sh = BwdShape<DK, DV>;
    constexpr int ROWS = Sh::ROWS, RG = Sh::RG, NCG = Sh::NCG;
    __shared__ BwdLds<DK, DV> L;
    const int bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
    const int cg = threadIdx.x % NCG, rg = threadIdx.x / NCG;
    const int64_t nck = (a.T + kCkpt - 1) / kCkpt;
    floatx4 dS[ROWS], sc[ROWS], s[ROWS];
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int c = rg + RG * i;
        dS[i] = a.dST ? *reinterpret_cast<const floatx4 *>(a.dST + ((int64_t)bh * DK + c) * DV + 4 * cg)
                      : floatx4{0, 0, 0, 0};
    }
    for (int64_t j = nck - 1; j >= 0; --j) {
        const int64_t t0 = j * kCkpt, t1 = t0 + kCkpt < a.T ? t0 + kCkpt : a.T;
        const float *src = a.ckpt + ((int64_t)bh * nck + j) * DK * DV;
#pragma unroll
        for (int i = 0; i < ROWS; ++i)
            sc[i] = *reinterpret_cast<const floatx4 *>(src + (rg + RG * i) * DV + 4 * cg);
        for (int64_t t = t1 - 1; t >= t0; --t) {
            // the state before token t, from the checkpoint
#pragma unroll
            for (int i = 0; i < ROWS; ++i) s[i] = sc[i];
            for (int64_t tau = t0; tau < t; ++tau)
                fwd_step<T, DK, DV>(L, a, ((int64_t)b * a.T + tau) * a.H + h, s);

            const int64_t row = ((int64_t)b * a.T + t) * a.H + h;
            load_token<T, DK, DV>(L, a, row, true);
            __syncthreads();
            const floatx4 vv = {L.v[4 * cg], L.v[4 * cg + 1], L.v[4 * cg + 2], L.v[4 * cg + 3]};
            const floatx4 dov = {L.dout[4 * cg], L.dout[4 * cg + 1], L.dout[4 * cg + 2],
                                 L.dout[4 * cg + 3]};
            const float bt = L.beta;
            // w = S'^T k, u = beta (v - w)
            floatx4 wp = {0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < ROWS; ++i) {
                const int c = rg + RG * i;
                wp += (L.a[c] * s[i]) * L.k[c];
            }
            const floatx4 w = row_sum<DK, DV>(L, wp, 0);
            const floatx4 u = bt * (vv - w);
            // dS += q do^T;  dq = S_t do;  du = dS^T k
            floatx4 dup = {0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < ROWS; ++i) {
                const int c = rg + RG * i;
                dS[i] += L.q[c] * dov;
                const floatx4 st = L.a[c] * s[i] + L.k[c] * u;
                const float dqc = col_sum<NCG>(dot4(st, dov));
                if (cg == 0) a.dq[row * DK + c] = dqc;
                dup += dS[i] * L.k[c];
            }
            const floatx4 du = row_sum<DK, DV>(L, dup, 1);
            // dbeta, dv (one row group writes), dw
            if (rg == 0) {
                const float db = col_sum<NCG>(dot4(du, vv - w));
                if (cg == 0) a.dbeta[row] = db;
                *reinterpret_cast<floatx4 *>(a.dv + row * DV + 4 * cg) = bt * du;
            }
            const floatx4 dw = -bt * du;
            // dk = dS u + S' dw;  dS' = dS + k dw^T;  dg = a * rowsum(S dS');  dS = a dS'
#pragma unroll
            for (int i = 0; i < ROWS; ++i) {
                const int c = rg + RG * i;
                const float ac = L.a[c];
                const floatx4 sp = ac * s[i];
                const float dkc = col_sum<NCG>(dot4(dS[i], u) + dot4(sp, dw));
                const floatx4 dsp = dS[i] + L.k[c] * dw;
                const float dac = col_sum<NCG>(dot4(s[i], dsp));
                if (cg == 0) {
                    a.dk[row * DK + c] = dkc;
                    a.dg[row * DK + c] = ac * dac;
                }
                dS[i] = ac * dsp;
            }
            __syncthreads();                     // LDS inputs are rewritten next
        }
    }
    if (a.dS0) {
#pragma unroll
        for (int i = 0; i < ROWS; ++i)
            *reinterpret_cast<floatx4 *>(a.dS0 + ((int64_t)bh * DK + rg + RG * i) * DV + 4 * cg) = dS[i];
    }
}

size_t bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int dk, int dv) {
    const int64_t nck = (T + kCkpt - 1) / kCkpt;
    return (size_t)B * H * nck * dk * dv * sizeof(float);
}

template <typename T, int DK, int DV>
static hipError_t bwd_inst(const BwdArgs &a, int nbh, hipStream_t s) {
    constexpr int TPB = BwdShape<DK, DV>::TPB;
    hipLaunchKernelGGL((bwd_ckpt_kernel<T, DK, DV>), dim3(nbh), dim3(TPB), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_kernel<T, DK, DV>), dim3(nbh), dim3(TPB), 0, s, a);
    return hipGetLastError();
}

template <typename T, int DK>
static hipError_t bwd_dv(const BwdArgs &a, int nbh, int dv, hipStream_t s) {
    switch (dv) {
    case 32: return bwd_inst<T, DK, 32>(a, nbh, s);
    case 64: return bwd_inst<T, DK, 64>(a, nbh, s);
    case 128: return bwd_inst<T, DK, 128>(a, nbh, s);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
static hipError_t bwd_dk(const BwdArgs &a, int nbh, int dk, int dv, hipStream_t s) {
    switch (dk) {
    case 32: return bwd_dv<T, 32>(a, nbh, dv, s);
    case 64: return bwd_dv<T, 64>(a, nbh, dv, s);
    case 128: return bwd_dv<T, 128>(a, nbh, dv, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_chunk_bwd(const void *q, const void *k, const void *v, const float *g,
                            const void *beta, const float *S0, const void *dout, const float *dST,
                            float *dq, float *dk_, float *dv_, float *dg, float *dbeta, float *dS0,
                            float *ckpt, int64_t B, int64_t T, int64_t H, int dk, int dv,
                            int is_bf16, hipStream_t s) {
    BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.dout = dout;
    a.g = g; a.S0 = S0; a.dST = dST; a.ckpt = ckpt;
    a.dq = dq; a.dk = dk_; a.dv = dv_; a.dg = dg; a.dbeta = dbeta; a.dS0 = dS0;
    a.T = T; a.H = (int)H;
    const int nbh = (int)(B * H);
    return is_bf16 ? bwd_dk<bf16>(a, nbh, dk, dv, s) : bwd_dk<float>(a, nbh, dk, dv, s);
}

}  // namespace kda
