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
// Every value column of S evolves on its own (w, u, du and dv are per
// column), so a chain's dv columns split over workgroups of NB = 32 columns;
// the per-row gradients dq, dk, dg and dbeta are sums over columns, written
// per slice and added in a fixed order by a last small kernel.
//
// A first pass stores the state before every kSeg-th token.  The reverse
// pass takes the segments from last to first: it stages the segment's inputs
// in LDS, runs the segment forward from its checkpoint keeping the kSeg
// states in registers (a thread holds float4 column groups of ROWS rows) and
// w, u per token in LDS, then walks the segment's tokens backwards.  Row
// sums reduce across the column lanes of a wave with lane exchanges, column
// sums across row groups through LDS: one barrier per forward step and one
// per reverse step.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kSeg = 8;                          // tokens per checkpoint segment
constexpr int kBwdCols = 32;                     // value columns per workgroup

template <int DK> struct BwdShape {
    static constexpr int NB = kBwdCols;
    static constexpr int NCG = NB / 4;           // float4 column groups
    static constexpr int TPB = 256;
    static constexpr int RG = TPB / NCG;         // row groups
    static constexpr int ROWS = DK / RG;         // rows per thread
    static constexpr int NWV = TPB / 64;
    static_assert(ROWS >= 1 && DK % RG == 0, "backward shape");
};

struct BwdArgs {
    const void *q, *k, *v, *beta, *dout;
    const float *g, *S0, *dST;
    float *ckpt;                                 // [nbh][nslice][nseg][DK][NB]
    float *part;                                 // per-slice row gradients when nslice > 1
    float *dq, *dk, *dv, *dg, *dbeta, *dS0;
    int64_t T, nrows;                            // nrows = B T H token rows
    int H, DV, nslice;
};

template <typename T> __device__ __forceinline__ float ldx(const void *p, int64_t i) {
    return to_f32(static_cast<const T *>(p)[i]);
}

template <int DK> struct BwdLds {
    float a[kSeg][DK], k[kSeg][DK], q[kSeg][DK];
    float v[kSeg][kBwdCols], dout[kSeg][kBwdCols];
    float w[kSeg][kBwdCols], u[kSeg][kBwdCols];
    float beta[kSeg];
    floatx4 red[2][BwdShape<DK>::NWV][BwdShape<DK>::NCG];
};

// Stage tokens t0 .. t0 + n - 1 of the chain (this slice's columns of v, do).
template <typename T, int DK>
__device__ __forceinline__ void load_segment(BwdLds<DK> &L, const BwdArgs &a, int64_t rowbase,
                                             int64_t t0, int n, int col0, bool with_read) {
    const int tid = threadIdx.x;
    for (int e = tid; e < n * DK; e += BwdShape<DK>::TPB) {
        const int i = e / DK, c = e % DK;
        const int64_t row = rowbase + (t0 + i) * a.H;
        L.a[i][c] = expf(a.g[row * DK + c]);
        L.k[i][c] = ldx<T>(a.k, row * DK + c);
        if (with_read) L.q[i][c] = ldx<T>(a.q, row * DK + c);
    }
    for (int e = tid; e < n * kBwdCols; e += BwdShape<DK>::TPB) {
        const int i = e / kBwdCols, n_ = e % kBwdCols;
        const int64_t row = rowbase + (t0 + i) * a.H;
        L.v[i][n_] = ldx<T>(a.v, row * a.DV + col0 + n_);
        if (with_read) L.dout[i][n_] = ldx<T>(a.dout, row * a.DV + col0 + n_);
    }
    if (tid < n) L.beta[tid] = ldx<T>(a.beta, rowbase + (t0 + tid) * a.H);
}

// Sum over all rows of a per-thread float4 partial (one column group); every
// thread of that column group receives the total.  Buffers alternate, so
// consecutive sums need one barrier each.
template <int DK>
__device__ __forceinline__ floatx4 row_sum(BwdLds<DK> &L, floatx4 x, int buf) {
    using Sh = BwdShape<DK>;
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

// Sum over the column groups (lanes of one row group); every lane receives it.
template <int NCG> __device__ __forceinline__ float col_sum(float x) {
#pragma unroll
    for (int m = 1; m < NCG; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

__device__ __forceinline__ float dot4(floatx4 x, floatx4 y) {
    return x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
}
__device__ __forceinline__ floatx4 lds4(const float *p) { return *reinterpret_cast<const floatx4 *>(p); }

// One forward step of segment token i on the register state s; w and u of
// the token are left in LDS.  `buf` selects the reduction buffer.
template <int DK>
__device__ __forceinline__ void fwd_step(BwdLds<DK> &L, int i, floatx4 (&s)[BwdShape<DK>::ROWS],
                                         int buf) {
    using Sh = BwdShape<DK>;
    const int cg = threadIdx.x % Sh::NCG, rg = threadIdx.x / Sh::NCG;
    floatx4 wp = {0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < Sh::ROWS; ++r) {
        const int c = rg + Sh::RG * r;
        s[r] *= L.a[i][c];
        wp += s[r] * L.k[i][c];
    }
    const floatx4 w = row_sum<DK>(L, wp, buf);
    const floatx4 u = L.beta[i] * (lds4(&L.v[i][4 * cg]) - w);
    if (rg == 0) {
        *reinterpret_cast<floatx4 *>(&L.w[i][4 * cg]) = w;
        *reinterpret_cast<floatx4 *>(&L.u[i][4 * cg]) = u;
    }
#pragma unroll
    for (int r = 0; r < Sh::ROWS; ++r) s[r] += L.k[i][rg + Sh::RG * r] * u;
}

// block -> (chain, column slice)
struct BwdBlock {
    int bh, b, h, slice, col0;
};
__device__ __forceinline__ BwdBlock bwd_block(const BwdArgs &a) {
    BwdBlock k;
    k.bh = blockIdx.x / a.nslice;
    k.slice = blockIdx.x % a.nslice;
    k.b = k.bh / a.H;
    k.h = k.bh % a.H;
    k.col0 = k.slice * kBwdCols;
    return k;
}

template <typename T, int DK>
__global__ __launch_bounds__(256) void bwd_ckpt_kernel(BwdArgs a) {
    using Sh = BwdShape<DK>;
    __shared__ BwdLds<DK> L;
    const BwdBlock blk = bwd_block(a);
    const int cg = threadIdx.x % Sh::NCG, rg = threadIdx.x / Sh::NCG;
    const int64_t nseg = (a.T + kSeg - 1) / kSeg;
    const int64_t rowbase = (int64_t)blk.b * a.T * a.H + blk.h;
    float *ck = a.ckpt + ((int64_t)blk.bh * a.nslice + blk.slice) * nseg * DK * kBwdCols;
    floatx4 s[Sh::ROWS];
#pragma unroll
    for (int r = 0; r < Sh::ROWS; ++r) {
        const int c = rg + Sh::RG * r;
        s[r] = a.S0 ? lds4(a.S0 + ((int64_t)blk.bh * DK + c) * a.DV + blk.col0 + 4 * cg)
                    : floatx4{0, 0, 0, 0};
    }
    for (int64_t j = 0; j < nseg; ++j) {
        const int64_t t0 = j * kSeg;
        const int n = (int)(a.T - t0 < kSeg ? a.T - t0 : kSeg);
#pragma unroll
        for (int r = 0; r < Sh::ROWS; ++r)
            *reinterpret_cast<floatx4 *>(ck + (j * DK + rg + Sh::RG * r) * kBwdCols + 4 * cg) = s[r];
        __syncthreads();                         // the previous segment's inputs are consumed
        load_segment<T, DK>(L, a, rowbase, t0, n, blk.col0, false);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kSeg; ++i)
            if (i < n) fwd_step<DK>(L, i, s, i & 1);
    }
}

template <typename T, int DK>
__global__ __launch_bounds__(256) void bwd_kernel(BwdArgs a) {
    using Sh = BwdShape<DK>;
    constexpr int ROWS = Sh::ROWS, RG = Sh::RG, NCG = Sh::NCG;
    __shared__ BwdLds<DK> L;
    const BwdBlock blk = bwd_block(a);
    const int cg = threadIdx.x % NCG, rg = threadIdx.x / NCG;
    const int64_t nseg = (a.T + kSeg - 1) / kSeg;
    const int64_t rowbase = (int64_t)blk.b * a.T * a.H + blk.h;
    const float *ck = a.ckpt + ((int64_t)blk.bh * a.nslice + blk.slice) * nseg * DK * kBwdCols;
    floatx4 dS[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        const int c = rg + RG * r;
        dS[r] = a.dST ? lds4(a.dST + ((int64_t)blk.bh * DK + c) * a.DV + blk.col0 + 4 * cg)
                      : floatx4{0, 0, 0, 0};
    }
    for (int64_t j = nseg - 1; j >= 0; --j) {
        const int64_t t0 = j * kSeg;
        const int n = (int)(a.T - t0 < kSeg ? a.T - t0 : kSeg);
        __syncthreads();                         // the previous segment's inputs are consumed
        load_segment<T, DK>(L, a, rowbase, t0, n, blk.col0, true);
        // st[i]: the state before segment token i
        floatx4 st[kSeg][ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) st[0][r] = lds4(ck + (j * DK + rg + RG * r) * kBwdCols + 4 * cg);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kSeg; ++i) {
            if (i < n) {
                floatx4 s[ROWS];
#pragma unroll
                for (int r = 0; r < ROWS; ++r) s[r] = st[i][r];
                fwd_step<DK>(L, i, s, i & 1);
                if (i + 1 < kSeg) {
#pragma unroll
                    for (int r = 0; r < ROWS; ++r) st[i + 1][r] = s[r];
                }
            }
        }
        __syncthreads();                         // w and u of every segment token are in LDS
#pragma unroll
        for (int i = kSeg - 1; i >= 0; --i) {
            if (i < n) {
                const int64_t row = rowbase + (t0 + i) * a.H;
                const floatx4 vv = lds4(&L.v[i][4 * cg]), dov = lds4(&L.dout[i][4 * cg]);
                const floatx4 w = lds4(&L.w[i][4 * cg]), u = lds4(&L.u[i][4 * cg]);
                const float bt = L.beta[i];
                // dS += q do^T;  dq = S_t do;  du = dS^T k
                floatx4 dup = {0, 0, 0, 0};
                float dqr[ROWS];
#pragma unroll
                for (int r = 0; r < ROWS; ++r) {
                    const int c = rg + RG * r;
                    dS[r] += L.q[i][c] * dov;
                    const floatx4 stt = L.a[i][c] * st[i][r] + L.k[i][c] * u;
                    dqr[r] = col_sum<NCG>(dot4(stt, dov));
                    dup += dS[r] * L.k[i][c];
                }
                const floatx4 du = row_sum<DK>(L, dup, (i + 1) & 1);
                const floatx4 dw = -bt * du;
                float dkr[ROWS], dgr[ROWS];
#pragma unroll
                for (int r = 0; r < ROWS; ++r) {
                    const int c = rg + RG * r;
                    const float ac = L.a[i][c];
                    const floatx4 sp = ac * st[i][r];
                    dkr[r] = col_sum<NCG>(dot4(dS[r], u) + dot4(sp, dw));
                    const floatx4 dsp = dS[r] + L.k[i][c] * dw;
                    dgr[r] = ac * col_sum<NCG>(dot4(st[i][r], dsp));
                    dS[r] = ac * dsp;
                }
                // this slice's columns: dv; its share of the row sums
                if (rg == 0)
                    *reinterpret_cast<floatx4 *>(a.dv + row * a.DV + blk.col0 + 4 * cg) = bt * du;
                const float dbp = col_sum<NCG>(dot4(du, vv - w));
                if (cg == 0) {
                    float *oq, *ok, *og;
                    if (a.nslice == 1) {
                        oq = a.dq + row * DK; ok = a.dk + row * DK; og = a.dg + row * DK;
                    } else {
                        // this slice's partial row: dq, dk, dg (DK each), dbeta
                        float *p = a.part + ((int64_t)blk.slice * a.nrows + row) * (3 * DK + 1);
                        oq = p; ok = p + DK; og = p + 2 * DK;
                    }
#pragma unroll
                    for (int r = 0; r < ROWS; ++r) {
                        const int c = rg + RG * r;
                        oq[c] = dqr[r];
                        ok[c] = dkr[r];
                        og[c] = dgr[r];
                    }
                    if (rg == 0) {
                        if (a.nslice == 1) a.dbeta[row] = dbp;
                        else og[DK] = dbp;
                    }
                }
            }
        }
    }
    if (a.dS0) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
            *reinterpret_cast<floatx4 *>(a.dS0 + ((int64_t)blk.bh * DK + rg + RG * r) * a.DV +
                                         blk.col0 + 4 * cg) = dS[r];
    }
}

// dq, dk, dg, dbeta = the slices' partial rows added in slice order.
template <int DK>
__global__ __launch_bounds__(256) void bwd_sum_kernel(BwdArgs a) {
    constexpr int W = 3 * DK + 1;
    const int64_t total = a.nrows * W;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
        float acc = a.part[e];
        for (int sl = 1; sl < a.nslice; ++sl) acc += a.part[(int64_t)sl * total + e];
        const int64_t row = e / W;
        const int c = (int)(e - row * W);
        if (c < DK) a.dq[row * DK + c] = acc;
        else if (c < 2 * DK) a.dk[row * DK + c - DK] = acc;
        else if (c < 3 * DK) a.dg[row * DK + c - 2 * DK] = acc;
        else a.dbeta[row] = acc;
    }
}

static size_t bwd_ckpt_bytes(int64_t B, int64_t T, int64_t H, int dk, int dv) {
    const int64_t nseg = (T + kSeg - 1) / kSeg;
    return (size_t)B * H * nseg * dk * dv * sizeof(float);
}
static size_t bwd_part_bytes(int64_t B, int64_t T, int64_t H, int dk, int dv) {
    const int nslice = dv / kBwdCols;
    return nslice > 1 ? (size_t)nslice * B * T * H * (3 * dk + 1) * sizeof(float) : 0;
}

size_t bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int dk, int dv) {
    const size_t ck = (bwd_ckpt_bytes(B, T, H, dk, dv) + 255) / 256 * 256;
    return ck + bwd_part_bytes(B, T, H, dk, dv);
}

template <typename T, int DK>
static hipError_t bwd_inst(const BwdArgs &a, int64_t nbh, hipStream_t s) {
    const unsigned grid = (unsigned)(nbh * a.nslice);
    hipLaunchKernelGGL((bwd_ckpt_kernel<T, DK>), dim3(grid), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_kernel<T, DK>), dim3(grid), dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess || a.nslice == 1) return e;
    int64_t blocks = (a.nrows * (3 * DK + 1) + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL((bwd_sum_kernel<DK>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <typename T>
static hipError_t bwd_dk(const BwdArgs &a, int64_t nbh, int dk, hipStream_t s) {
    switch (dk) {
    case 32: return bwd_inst<T, 32>(a, nbh, s);
    case 64: return bwd_inst<T, 64>(a, nbh, s);
    case 128: return bwd_inst<T, 128>(a, nbh, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_chunk_bwd(const void *q, const void *k, const void *v, const float *g,
                            const void *beta, const float *S0, const void *dout, const float *dST,
                            float *dq, float *dk_, float *dv_, float *dg, float *dbeta, float *dS0,
                            float *ws, int64_t B, int64_t T, int64_t H, int dk, int dv,
                            int is_bf16, hipStream_t s) {
    if (dv % kBwdCols) return hipErrorInvalidValue;
    BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.dout = dout;
    a.g = g; a.S0 = S0; a.dST = dST;
    a.ckpt = ws;
    a.part = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) +
                                       (bwd_ckpt_bytes(B, T, H, dk, dv) + 255) / 256 * 256);
    a.dq = dq; a.dk = dk_; a.dv = dv_; a.dg = dg; a.dbeta = dbeta; a.dS0 = dS0;
    a.T = T; a.nrows = B * T * H; a.H = (int)H; a.DV = dv; a.nslice = dv / kBwdCols;
    return is_bf16 ? bwd_dk<bf16>(a, B * H, dk, s) : bwd_dk<float>(a, B * H, dk, s);
}

}  // namespace kda
