// Chunkwise reverse mode of the KDA recurrence: 16-token chunks, every product
// on the fp32 matrix cores (v_mfma_f32_16x16x4f32), so the gradients keep fp32
// accuracy.
//
// The forward step is the one of "Kimi K3 internal structure analysis",
// section "Sequence mixing: 3 KDA layers per global MLA layer" (retention,
// delta-rule write, read after the write).  The pages say nothing of
// training; the reverse mode below is derived from the chunk form of that
// step.  For one chain and one chunk of C = 16 tokens, with S the state
// entering it, b_r the running sum of g inside the chunk, m = b_7 and
// b_C = b_15 (per key channel):
//     K~ = k e^b, Q~ = q e^b, K^ = k e^{b_C - b}            (all <= 1)
//     K' = k e^{b-m}, Q' = q e^{b-m}, K" = k e^{m-b}         (<= e^40 each)
//     At = K' K"^T,  A = strict_lower(Diag(beta) At),  P = lower(Q' K"^T)
//     X  = (I + A)^-1,  W = V - K~ S,  U = X Diag(beta) W
//     O  = Q~ S + P U,  S_next = Diag(e^{b_C}) S + K^^T U
// Referencing the pair factors to the middle token keeps each operand within
// e^{+-40} when the 16-token decay sum is >= -80 (the gate floor's bound), so
// K' K"^T = sum k k e^{b_r - b_s} is formed with no overflow.
//
// Reverse, given dO and dN = dL/dS_next:
//     dU = P^T dO + K^ dN,   dW = Diag(beta) X^T dU,   dv = dW
//     dS = Diag(e^{b_C}) dN + Q~^T dO - K~^T dW                (to the previous chunk)
//     dT = dU W^T,   dX = dT Diag(beta),   dbeta_s += sum_r X_rs dT_rs
//     dA = strict_lower(-X^T dX X^T),   dbeta_r += sum_s dA_rs At_rs,   dAt = Diag(beta) dA
//     dP = lower(dO U^T)
//     dQ' = dP K",  dK' = dAt K",  dK" = dAt^T K' + dP^T Q'
//     dQ~ = dO S^T,  dK~ = -dW S^T,  dK^ = U dN^T
//     dq = dQ~ e^b + dQ' e^{b-m}
//     dk = dK~ e^b + dK^ e^{b_C-b} + dK' e^{b-m} + dK" e^{m-b}
//     db = dQ~ Q~ + dK~ K~ - dK^ K^ + dQ' Q' + dK' K' - dK" K"   (per token)
//     db_C += sum_r dK^ K^ + e^{b_C} rowsum(S * dN)
//     dg_t = sum_{r >= t} db_r
// (m cancels from every output, so its gradient is zero and is not formed.)
//
// Four launches:
//   cb_prep_kernel   per chunk: At, P, X (16x16 each) and the decayed
//                    operands K~, K^, Q~, e^{b_C} to the workspace
//   cb_fwd_kernel    per (chain, 32-column slice), chunks in order: the state
//                    entering each even chunk and W of every chunk to the
//                    workspace
//   cb_bwd_kernel    per (chain, slice), chunks in reverse: dN leaving each
//                    odd chunk (and the last), dU of every chunk, and
//                    d(initial state)
//   cb_grad_kernel   one workgroup per chunk pair, all pairs at once: every
//                    token gradient from (S, dN, W, dU, At, X), the pair's
//                    state products in one sweep over its two stored tiles
// The two passes carry their state slice in MFMA accumulator registers (lane
// l holds rows 4(l/16)+i, column l%16 of each 16x16 tile), which is also a
// valid B operand of the next product once the contraction index is taken in
// the same order on both operands.
#include <math.h>
#include <stdint.h>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kCB = 16;                          // tokens per chunk
constexpr int kCbMat = 3 * kCB * kCB;            // X, P, At per chunk

// e^x with the hardware base-2 exponential.  Every exponent here is a
// difference of cumulative log-decays inside one 16-token chunk, or such a sum
// from the chunk start: within [-80, 80] under the gate floor, so the result
// is a normal fp32 number, within a few ulp of expf (the rounding of x log2 e
// adds at most |x| 2^-24 to the exponent).
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

struct CbArgs {
    const void *q, *k, *v, *beta, *dout;
    const float *g, *S0, *dST;
    float *dq, *dk, *dv, *dg, *dbeta, *dS0;
    float *st;                                   // [nbh][np][DK][DV]  state entering chunk 2p
    float *dn;                                   // [nbh][np][DK][DV]  gradient leaving chunk 2p+1
                                                 //                    (chunk 2p when it is the last)
    float *mat;                                  // [nbh][nc][3][16][16]  X, P, At
    float *ops;                                  // [nbh][nc][cb_ops_floats(DK)]  decayed operands
    float *w;                                    // [nbh][nc][16][DV]
    float *du;                                   // [nbh][nc][16][DV]
    float *sfinal;                               // cb_fwd_kernel: the state after the last
                                                 // chunk, [nbh][DK][DV] (null: not written)
    void *o;                                     // cb_fwd_kernel<.., true>: the outputs
                                                 // O = Q~ S + P U, [B, tseq, H, DV] in T
    const int *slots;                            // cb_fwd_kernel<.., true>: with a slot table
    int64_t n_slots;                             // the states are rows slots[b] H + h of a pool
                                                 // (a slot outside it skips the sequence)
    int64_t T;                                   // tokens of this launch (a segment)
    int64_t tseq, toff;                          // tokens per sequence in memory; first token
    int H, DV, nc, nsl, np;                      // np = chunk pairs = ceil(nc / 2)
};

// Decayed operands of one chunk, each once, channel-major: K~^T, K^^T, Q~^T
// [DK][16] and e^{b_C} [DK].  The state passes copy them to LDS as they are,
// and also transpose K~ (forward pass) or K^ (reverse pass) into token rows
// while staging.
__host__ __device__ constexpr int cb_ops_floats(int DK) { return 49 * DK; }
enum { kOpKtT = 0, kOpKhT = 16, kOpQtT = 32, kOpEbc = 48 };  // x DK

template <typename T> __device__ __forceinline__ float cb_ld(const void *p, int64_t i) {
    return to_f32(static_cast<const T *>(p)[i]);
}

__device__ __forceinline__ floatx4 mfma1(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Row of the launch's token 0 (token toff of the sequence) of chain bh in the
// [B, tseq, H] token layout; token t of the launch is row cb_rowbase + t * H.
__device__ __forceinline__ int64_t cb_rowbase(const CbArgs &a, int64_t bh) {
    return (bh / a.H) * a.tseq * a.H + bh % a.H + a.toff * a.H;
}

// The 16 values of one channel over the chunk's tokens: element `off` of
// rows rowbase + (t0 + r) H, row length `ld`.  Padded tokens past the end
// (r >= n) read the last valid row and are then zeroed, so every load is
// unconditional and all 16 are in flight together.
template <typename T>
__device__ __forceinline__ void cb_load16(const void *p, int64_t rowbase, int64_t t0, int n, int H,
                                          int ld, int off, float (&x)[kCB]) {
#pragma unroll
    for (int r = 0; r < kCB; ++r) {
        const int rr = r < n ? r : n - 1;
        x[r] = cb_ld<T>(p, (rowbase + (t0 + rr) * H) * ld + off);
    }
#pragma unroll
    for (int r = 0; r < kCB; ++r) x[r] = r < n ? x[r] : 0.f;
}

// Running log-decay of one key channel over the chunk (g = 0 past the end).
__device__ __forceinline__ void cb_cumsum(const float (&gv)[kCB], float (&b)[kCB]) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < kCB; ++r) {
        s += gv[r];
        b[r] = s;
    }
}

// ---------------------------------------------------------------------------
// At, P, X and the decayed operands of one chunk.  Four waves: thread t <
// 2 DK takes channel t % DK over tokens 8 (t / DK) .. +7 (the two halves
// exchange their decay totals through LDS); then wave 0 forms At and X,
// wave 1 forms P.
// ---------------------------------------------------------------------------
template <typename T, int DK>
__global__ __launch_bounds__(256) void cb_prep_kernel(CbArgs a) {
    constexpr int LD = DK + 4, HT = kCB / 2;
    __shared__ __attribute__((aligned(16))) float Kp[kCB][LD], Kpp[kCB][LD], Qp[kCB][LD];
    __shared__ float tot[2][DK];
    __shared__ float Am[kCB][kCB + 1], bet[kCB];
    const int64_t unit = blockIdx.x;
    const int64_t bh = unit / a.nc;
    const int c = (int)(unit % a.nc);
    const int64_t t0 = (int64_t)c * kCB;
    const int n = (int)(a.T - t0 < kCB ? a.T - t0 : kCB);
    const int tid = threadIdx.x, lane = tid & 63, j = lane & 15, g4 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t rb = cb_rowbase(a, bh);
    const int ch = tid % DK, half = tid / DK;
    float gv[HT], kv[HT], qv[HT], b[HT];
    if (tid < 2 * DK) {
#pragma unroll
        for (int r = 0; r < HT; ++r) {
            const int tr = HT * half + r, rr = tr < n ? tr : n - 1;
            const int64_t off = (rb + (t0 + rr) * a.H) * DK + ch;
            gv[r] = a.g[off];
            kv[r] = cb_ld<T>(a.k, off);
            qv[r] = cb_ld<T>(a.q, off);
        }
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < HT; ++r) {
            const bool ok = HT * half + r < n;
            gv[r] = ok ? gv[r] : 0.f;
            kv[r] = ok ? kv[r] : 0.f;
            qv[r] = ok ? qv[r] : 0.f;
            sum += gv[r];
            b[r] = sum;
        }
        tot[half][ch] = sum;
    }
    if (tid < kCB) bet[tid] = (tid < n) ? cb_ld<T>(a.beta, rb + (t0 + tid) * a.H) : 0.f;
    __syncthreads();
    if (tid < 2 * DK) {
        const float m = tot[0][ch];                       // b_7
        const float bc = tot[0][ch] + tot[1][ch];         // b_15
        const float base = half ? m : 0.f;
        float *op = a.ops + unit * cb_ops_floats(DK);
        float kt[HT], kh[HT], qt[HT];
#pragma unroll
        for (int r = 0; r < HT; ++r) {
            const int tr = HT * half + r;
            const float br = base + b[r];
            const float e = exp_hw(br - m), ei = exp_hw(m - br), eb = exp_hw(br);
            Kp[tr][ch] = kv[r] * e;
            Kpp[tr][ch] = kv[r] * ei;
            Qp[tr][ch] = qv[r] * e;
            kt[r] = kv[r] * eb;
            kh[r] = kv[r] * exp_hw(bc - br);
            qt[r] = qv[r] * eb;
        }
#pragma unroll
        for (int r = 0; r < HT; r += 4) {
            const int tr = HT * half + r;
            *reinterpret_cast<floatx4 *>(op + kOpKtT * DK + ch * kCB + tr) =
                floatx4{kt[r], kt[r + 1], kt[r + 2], kt[r + 3]};
            *reinterpret_cast<floatx4 *>(op + kOpKhT * DK + ch * kCB + tr) =
                floatx4{kh[r], kh[r + 1], kh[r + 2], kh[r + 3]};
            *reinterpret_cast<floatx4 *>(op + kOpQtT * DK + ch * kCB + tr) =
                floatx4{qt[r], qt[r + 1], qt[r + 2], qt[r + 3]};
        }
        if (half == 0) op[kOpEbc * DK + ch] = exp_hw(bc);
    }
    __syncthreads();
    float *mat = a.mat + unit * kCbMat;          // X, P, At
    if (wave == 0) {
        floatx4 at = {0, 0, 0, 0};
        tile_mma<float>(at, &Kp[0][0], LD, &Kpp[0][0], LD, DK, lane);   // at[i] = At[4g4+i][j]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g4 + i;
            const float atv = (j < r) ? at[i] : 0.f;  // selects: the masked entries may be large
            mat[2 * kCB * kCB + r * kCB + j] = atv;
            Am[r][j] = bet[r] * atv;
        }
    } else if (wave == 1) {
        floatx4 pp = {0, 0, 0, 0};
        tile_mma<float>(pp, &Qp[0][0], LD, &Kpp[0][0], LD, DK, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g4 + i;
            mat[kCB * kCB + r * kCB + j] = (j <= r) ? pp[i] : 0.f;
        }
    }
    __syncthreads();
    // X = (I + A)^-1 by forward substitution, one column per lane.
    if (tid < kCB) {
        float x[kCB];
#pragma unroll
        for (int r = 0; r < kCB; ++r) {
            float sacc = (r == tid) ? 1.f : 0.f;
#pragma unroll
            for (int q = 0; q < r; ++q) sacc -= Am[r][q] * x[q];
            x[r] = sacc;
            mat[r * kCB + tid] = sacc;
        }
    }
}

// block -> (chain, column slice); the slices of a chain share an XCD (and
// its L2) when the chain count is a multiple of 8.
__device__ __forceinline__ void cb_slice_block(const CbArgs &a, int64_t nbh, int64_t &bh, int &sl) {
    const int64_t x = blockIdx.x;
    if (nbh % 8 == 0) {
        bh = (x / (8 * a.nsl)) * 8 + x % 8;
        sl = (int)((x / 8) % a.nsl);
    } else {
        bh = x / a.nsl;
        sl = (int)(x % a.nsl);
    }
}

// Value columns per workgroup of the two state passes (two 16-column tiles).
constexpr int kCbNS = 32;
constexpr int kCbCT = kCbNS / 16;

// LDS of the two state passes, double-buffered over chunks.
template <int DK> struct alignas(16) CbPassLds {
    float rowm[2][kCB][DK + 4];                  // fwd: K~    bwd: K^          [token][channel]
    float colm1[2][DK][kCB + 4];                 // fwd: K^ T  bwd: Q~ T       [channel][token]
    float colm2[2][DK][kCB + 4];                 //            bwd: K~ T
    float ebc[2][DK];                            // e^{b_C}
    // pitches: rows 4 apart land 16 banks apart, so the accumulator-layout
    // accesses (row 4(l/16)+i, column l%16) of a wave hit distinct banks
    float vo[2][kCB][kCbNS + 4];                 // fwd: V slice  bwd: dO slice
    float X[2][kCB][kCB + 4];
    float P[2][kCB][kCB + 4];
    float bet[2][kCB];
    float red[4][kCB][kCbNS + 4];
};

// One chunk's inputs of a state pass, fetched into registers a chunk ahead
// of their use (the passes are sequential over chunks, so their load latency
// would otherwise be paid once per chunk).
template <int DK> struct CbStage {
    static constexpr int NF = (4 * DK + 255) / 256;   // float4 of one [16][DK] array per thread
    static constexpr int NV = kCB * kCbNS / 256;      // value (or dO) elements per thread
    floatx4 r1[NF], r2[NF], r3[NF], e;
    float vo[NV], x, p, bet;
};

__device__ __forceinline__ floatx4 ld4(const float *p) { return *reinterpret_cast<const floatx4 *>(p); }

// fwd: r1 = K~^T (staged as token rows), r2 = K^^T, and with outputs (OUT)
// r3 = Q~^T (staged as token rows) and P; bwd: r1 = K^^T (staged as token
// rows), r2 = Q~^T, r3 = K~^T.
// `vsrc` is v (fwd) or dO (bwd).
template <typename T, int DK, bool BWD, bool OUT = false>
__device__ __forceinline__ void cb_fetch(const CbArgs &a, const void *vsrc, int64_t bh, int64_t rb,
                                         int col0, int c, CbStage<DK> &st) {
    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)c * kCB;
    const int n = (int)(a.T - t0 < kCB ? a.T - t0 : kCB);
    const float *op = a.ops + (bh * a.nc + c) * cb_ops_floats(DK);
#pragma unroll
    for (int u = 0; u < CbStage<DK>::NF; ++u) {
        const int idx = tid + 256 * u;
        if (idx < 4 * DK) {
            st.r1[u] = ld4(op + (BWD ? kOpKhT : kOpKtT) * DK + 4 * idx);
            st.r2[u] = ld4(op + (BWD ? kOpQtT : kOpKhT) * DK + 4 * idx);
            if (BWD || OUT) st.r3[u] = ld4(op + (BWD ? kOpKtT : kOpQtT) * DK + 4 * idx);
        }
    }
    if (tid < DK / 4) st.e = ld4(op + kOpEbc * DK + 4 * tid);
#pragma unroll
    for (int u = 0; u < CbStage<DK>::NV; ++u) {
        const int e = tid + 256 * u, r = e / kCbNS, cc = e % kCbNS, rr = r < n ? r : n - 1;
        st.vo[u] = cb_ld<T>(vsrc, (rb + (t0 + rr) * a.H) * a.DV + col0 + cc);
    }
    const int r = tid >> 4, cc = tid & 15;
    const float *mc = a.mat + (bh * a.nc + c) * kCbMat;
    st.x = mc[r * kCB + cc];
    if (BWD || OUT) st.p = mc[kCB * kCB + r * kCB + cc];
    const int tb = (tid & 15) < n ? (tid & 15) : n - 1;
    st.bet = cb_ld<T>(a.beta, rb + (t0 + tb) * a.H);
}

// The forward pass with outputs stages Q~ in token rows over colm2, which
// only the reverse pass uses.
template <int DK> __device__ __forceinline__ float *cb_rowq(CbPassLds<DK> &L, int buf) {
    static_assert(2 * kCB * (DK + 4) <= 2 * DK * (kCB + 4), "Q~ rows fit over colm2");
    return &L.colm2[0][0][0] + buf * kCB * (DK + 4);
}

template <int DK, bool BWD, bool OUT = false>
__device__ __forceinline__ void cb_stage_to_lds(CbPassLds<DK> &L, const CbStage<DK> &st, int buf,
                                                int n) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < CbStage<DK>::NF; ++u) {
        const int idx = tid + 256 * u;
        if (idx < 4 * DK) {
            const int f = 4 * idx;                  // channel f / 16, tokens f % 16 ..
#pragma unroll
            for (int e = 0; e < 4; ++e) L.rowm[buf][f % kCB + e][f / kCB] = st.r1[u][e];
            *reinterpret_cast<floatx4 *>(&L.colm1[buf][f / kCB][f % kCB]) = st.r2[u];
            if (BWD) *reinterpret_cast<floatx4 *>(&L.colm2[buf][f / kCB][f % kCB]) = st.r3[u];
            if (OUT) {
                float *rq = cb_rowq(L, buf);
#pragma unroll
                for (int e = 0; e < 4; ++e) rq[(f % kCB + e) * (DK + 4) + f / kCB] = st.r3[u][e];
            }
        }
    }
    if (tid < DK / 4) *reinterpret_cast<floatx4 *>(&L.ebc[buf][4 * tid]) = st.e;
#pragma unroll
    for (int u = 0; u < CbStage<DK>::NV; ++u) {
        const int e = tid + 256 * u, r = e / kCbNS, cc = e % kCbNS;
        L.vo[buf][r][cc] = r < n ? st.vo[u] : 0.f;
    }
    const int r = tid >> 4, cc = tid & 15;
    L.X[buf][r][cc] = st.x;
    if (BWD || OUT) L.P[buf][r][cc] = st.p;
    if (tid < kCB) L.bet[buf][tid] = tid < n ? st.bet : 0.f;
}

// Chunks of register prefetch in the two state passes.  The passes' barriers
// wait for LDS only (lds_barrier), so loads stay in flight across them and
// the stores of states and W never hold a barrier up.  Two chunks ahead keep
// both passes at two waves per SIMD (at most 248 of the 512 registers of a
// lane); three push the reverse pass to one wave per SIMD and run slower.
constexpr int kCbAhead = 2;

// ---------------------------------------------------------------------------
// Forward state pass: the state entering every chunk, and W = V - K~ S.
// Wave w owns row tiles w*TPW .. of the workgroup's 32 value columns.
// ---------------------------------------------------------------------------
template <int DK> using CbAcc = floatx4[(DK / 16 + 3) / 4][kCbCT];

// LDS of the forward pass; with outputs (the prefill of shapes the other
// kernels do not take) a second cross-wave reduction for Q~ S.
template <int DK, bool OUT> struct CbFwdLds : CbPassLds<DK> {};
template <int DK> struct CbFwdLds<DK, true> : CbPassLds<DK> {
    float red2[4][kCB][kCbNS + 4];
};

template <typename T, int DK, bool OUT>
__device__ __forceinline__ void cb_fwd_step(const CbArgs &a, CbFwdLds<DK, OUT> &L, CbStage<DK> &stg,
                                            int c, int64_t bh, int64_t rb, int col0, int wave,
                                            CbAcc<DK> &s) {
    constexpr int RT = DK / 16, TPW = (RT + 3) / 4;
    const int lane = threadIdx.x & 63, j = lane & 15, g4 = lane >> 4;
    const int buf = c & 1;
    const int64_t t0 = (int64_t)c * kCB;
    const int n = (int)(a.T - t0 < kCB ? a.T - t0 : kCB);
    cb_stage_to_lds<DK, false, OUT>(L, stg, buf, n);
    cb_fetch<T, DK, false, OUT>(a, a.v, bh, rb, col0, c + kCbAhead < a.nc ? c + kCbAhead : a.nc - 1, stg);
    if constexpr (!OUT) {
        // the state entering each even chunk (the gradient kernel forms the odd ones)
        float *stc = a.st + ((bh * a.np + c / 2) * DK) * a.DV + col0 + j;
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int tt = wave * TPW + u;
            if (tt < RT && (c & 1) == 0) {
#pragma unroll
                for (int v = 0; v < kCbCT; ++v)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        stc[(int64_t)(16 * tt + 4 * g4 + i) * a.DV + 16 * v] = s[u][v][i];
            }
        }
    }
    lds_barrier();
    // this wave's rows of K~ S (and of Q~ S, with outputs)
    floatx4 wp[kCbCT], qp[kCbCT];
#pragma unroll
    for (int v = 0; v < kCbCT; ++v) wp[v] = qp[v] = floatx4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int tt = wave * TPW + u;
        if (tt < RT) {
            const floatx4 kt = ld4(&L.rowm[buf][j][16 * tt + 4 * g4]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int v = 0; v < kCbCT; ++v) wp[v] = mfma1(kt[i], s[u][v][i], wp[v]);
            if constexpr (OUT) {
                const floatx4 qt = ld4(cb_rowq<DK>(L, buf) + j * (DK + 4) + 16 * tt + 4 * g4);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int v = 0; v < kCbCT; ++v) qp[v] = mfma1(qt[i], s[u][v][i], qp[v]);
            }
        }
    }
#pragma unroll
    for (int v = 0; v < kCbCT; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            L.red[wave][4 * g4 + i][16 * v + j] = wp[v][i];
            if constexpr (OUT) L.red2[wave][4 * g4 + i][16 * v + j] = qp[v][i];
        }
    lds_barrier();
    const floatx4 xr = ld4(&L.X[buf][j][4 * g4]);
    floatx4 U[kCbCT];
#pragma unroll
    for (int v = 0; v < kCbCT; ++v) {
        const int cc = 16 * v + j;
        floatx4 W;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g4 + i;
            W[i] = L.vo[buf][r][cc] -
                   (L.red[0][r][cc] + L.red[1][r][cc] + L.red[2][r][cc] + L.red[3][r][cc]);
        }
        if constexpr (!OUT) {
            if (wave == 0) {
                float *wc = a.w + ((bh * a.nc + c) * kCB) * a.DV + col0 + cc;
#pragma unroll
                for (int i = 0; i < 4; ++i) wc[(int64_t)(4 * g4 + i) * a.DV] = W[i];
            }
        }
        // U = X Diag(beta) W
        U[v] = floatx4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) U[v] = mfma1(xr[i], L.bet[buf][4 * g4 + i] * W[i], U[v]);
        if constexpr (OUT) {
            // O = Q~ S + P U (rows past the end are not written)
            if (wave == 0) {
                floatx4 O;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * g4 + i;
                    O[i] = L.red2[0][r][cc] + L.red2[1][r][cc] + L.red2[2][r][cc] + L.red2[3][r][cc];
                }
                const floatx4 pr = ld4(&L.P[buf][j][4 * g4]);
#pragma unroll
                for (int i = 0; i < 4; ++i) O = mfma1(pr[i], U[v][i], O);
                T *oc = static_cast<T *>(a.o) + (rb + t0 * a.H) * a.DV + col0 + cc;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * g4 + i < n) oc[(int64_t)(4 * g4 + i) * a.H * a.DV] = from_f32<T>(O[i]);
            }
        }
    }
    // S <- Diag(e^{b_C}) S + K^^T U
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int tt = wave * TPW + u;
        if (tt < RT) {
            const floatx4 kh = ld4(&L.colm1[buf][16 * tt + j][4 * g4]);
#pragma unroll
            for (int v = 0; v < kCbCT; ++v) {
#pragma unroll
                for (int i = 0; i < 4; ++i) s[u][v][i] *= L.ebc[buf][16 * tt + 4 * g4 + i];
#pragma unroll
                for (int i = 0; i < 4; ++i) s[u][v] = mfma1(kh[i], U[v][i], s[u][v]);
            }
        }
    }
}

// Store this wave's tiles of the slice into a [B*H, DK, DV] state (the
// layout cb_load_state reads).
template <int DK>
__device__ __forceinline__ void cb_store_state(float *dst, int64_t bh, int DV, int col0, int wave,
                                               const CbAcc<DK> &s) {
    constexpr int RT = DK / 16, TPW = (RT + 3) / 4;
    const int lane = threadIdx.x & 63, j = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int tt = wave * TPW + u;
        if (tt < RT) {
#pragma unroll
            for (int v = 0; v < kCbCT; ++v)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dst[(bh * DK + 16 * tt + 4 * g4 + i) * DV + col0 + 16 * v + j] = s[u][v][i];
        }
    }
}

// Load (or zero) this wave's tiles of a [B*H, DK, DV] state for the slice.
template <int DK>
__device__ __forceinline__ void cb_load_state(const float *src, int64_t bh, int DV, int col0,
                                              int wave, CbAcc<DK> &s) {
    constexpr int RT = DK / 16, TPW = (RT + 3) / 4;
    const int lane = threadIdx.x & 63, j = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int tt = wave * TPW + u;
#pragma unroll
        for (int v = 0; v < kCbCT; ++v)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s[u][v][i] = (src && tt < RT)
                                 ? src[(bh * DK + 16 * tt + 4 * g4 + i) * DV + col0 + 16 * v + j] : 0.f;
    }
}

template <typename T, int DK, bool OUT = false>
__global__ __launch_bounds__(256) void cb_fwd_kernel(CbArgs a, int64_t nbh) {
    __shared__ CbFwdLds<DK, OUT> L;
    int64_t bh;
    int sl;
    cb_slice_block(a, nbh, bh, sl);
    const int64_t rb = cb_rowbase(a, bh);
    const int col0 = sl * kCbNS;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // row of the chain's states: bh, or its slot's row of a state pool
    int64_t srow = bh;
    if (OUT && a.slots) {
        const int slot = a.slots[bh / a.H];
        if (slot < 0 || slot >= a.n_slots) return;
        srow = (int64_t)slot * a.H + bh % a.H;
    }
    CbAcc<DK> s;
    cb_load_state<DK>(a.S0, srow, a.DV, col0, wave, s);
    CbStage<DK> stg[kCbAhead];
#pragma unroll
    for (int q = 0; q < kCbAhead; ++q)
        cb_fetch<T, DK, false, OUT>(a, a.v, bh, rb, col0, q < a.nc ? q : a.nc - 1, stg[q]);
    for (int c0 = 0; c0 < a.nc; c0 += kCbAhead) {
#pragma unroll
        for (int q = 0; q < kCbAhead; ++q)
            if (c0 + q < a.nc) cb_fwd_step<T, DK, OUT>(a, L, stg[q], c0 + q, bh, rb, col0, wave, s);
    }
    if (a.sfinal) cb_store_state<DK>(a.sfinal, srow, a.DV, col0, wave, s);
}

// ---------------------------------------------------------------------------
// Reverse state pass: dN of every chunk, dU, and d(initial state).
// ---------------------------------------------------------------------------
template <typename T, int DK>
__device__ __forceinline__ void cb_bwd_step(const CbArgs &a, CbPassLds<DK> &L, CbStage<DK> &stg,
                                            int c, int64_t bh, int64_t rb, int col0, int wave,
                                            CbAcc<DK> &d) {
    constexpr int RT = DK / 16, TPW = (RT + 3) / 4;
    const int lane = threadIdx.x & 63, j = lane & 15, g4 = lane >> 4;
    const int buf = c & 1;
    const int64_t t0 = (int64_t)c * kCB;
    const int n = (int)(a.T - t0 < kCB ? a.T - t0 : kCB);
    cb_stage_to_lds<DK, true>(L, stg, buf, n);
    cb_fetch<T, DK, true>(a, a.dout, bh, rb, col0, c >= kCbAhead ? c - kCbAhead : 0, stg);
    // the gradient leaving each odd chunk, and the last chunk (the gradient
    // kernel forms those of the other even chunks)
    float *dnc = a.dn + ((bh * a.np + c / 2) * DK) * a.DV + col0 + j;
    const bool keep = (c & 1) == 1 || c == a.nc - 1;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int tt = wave * TPW + u;
        if (tt < RT && keep) {
#pragma unroll
            for (int v = 0; v < kCbCT; ++v)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dnc[(int64_t)(16 * tt + 4 * g4 + i) * a.DV + 16 * v] = d[u][v][i];
        }
    }
    lds_barrier();
    // this wave's rows of K^ dN (wave 0 adds P^T dO)
    floatx4 up[kCbCT];
#pragma unroll
    for (int v = 0; v < kCbCT; ++v) up[v] = floatx4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int tt = wave * TPW + u;
        if (tt < RT) {
            const floatx4 kh = ld4(&L.rowm[buf][j][16 * tt + 4 * g4]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int v = 0; v < kCbCT; ++v) up[v] = mfma1(kh[i], d[u][v][i], up[v]);
        }
    }
    if (wave == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float pv = L.P[buf][4 * g4 + i][j];
#pragma unroll
            for (int v = 0; v < kCbCT; ++v) up[v] = mfma1(pv, L.vo[buf][4 * g4 + i][16 * v + j], up[v]);
        }
    }
#pragma unroll
    for (int v = 0; v < kCbCT; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) L.red[wave][4 * g4 + i][16 * v + j] = up[v][i];
    lds_barrier();
    floatx4 dW[kCbCT];
#pragma unroll
    for (int v = 0; v < kCbCT; ++v) {
        const int cc = 16 * v + j;
        floatx4 dU;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g4 + i;
            dU[i] = L.red[0][r][cc] + L.red[1][r][cc] + L.red[2][r][cc] + L.red[3][r][cc];
        }
        if (wave == 0) {
            float *duc = a.du + ((bh * a.nc + c) * kCB) * a.DV + col0 + cc;
#pragma unroll
            for (int i = 0; i < 4; ++i) duc[(int64_t)(4 * g4 + i) * a.DV] = dU[i];
        }
        // dW = Diag(beta) X^T dU, kept negated: it enters with K~^T
        dW[v] = floatx4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) dW[v] = mfma1(L.X[buf][4 * g4 + i][j], dU[i], dW[v]);
#pragma unroll
        for (int i = 0; i < 4; ++i) dW[v][i] *= -L.bet[buf][4 * g4 + i];
    }
    // dN <- Diag(e^{b_C}) dN + Q~^T dO - K~^T dW
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int tt = wave * TPW + u;
        if (tt < RT) {
            const floatx4 qt = ld4(&L.colm1[buf][16 * tt + j][4 * g4]);
            const floatx4 kt = ld4(&L.colm2[buf][16 * tt + j][4 * g4]);
#pragma unroll
            for (int v = 0; v < kCbCT; ++v) {
#pragma unroll
                for (int i = 0; i < 4; ++i) d[u][v][i] *= L.ebc[buf][16 * tt + 4 * g4 + i];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    d[u][v] = mfma1(qt[i], L.vo[buf][4 * g4 + i][16 * v + j], d[u][v]);
#pragma unroll
                for (int i = 0; i < 4; ++i) d[u][v] = mfma1(kt[i], dW[v][i], d[u][v]);
            }
        }
    }
}

template <typename T, int DK>
__global__ __launch_bounds__(256) void cb_bwd_kernel(CbArgs a, int64_t nbh) {
    constexpr int RT = DK / 16, TPW = (RT + 3) / 4;
    __shared__ CbPassLds<DK> L;
    int64_t bh;
    int sl;
    cb_slice_block(a, nbh, bh, sl);
    const int64_t rb = cb_rowbase(a, bh);
    const int col0 = sl * kCbNS;
    const int lane = threadIdx.x & 63, j = lane & 15, g4 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    CbAcc<DK> d;
    cb_load_state<DK>(a.dST, bh, a.DV, col0, wave, d);
    CbStage<DK> stg[kCbAhead];
#pragma unroll
    for (int q = 0; q < kCbAhead; ++q)
        cb_fetch<T, DK, true>(a, a.dout, bh, rb, col0, a.nc - 1 - q >= 0 ? a.nc - 1 - q : 0, stg[q]);
    for (int c0 = a.nc - 1; c0 >= 0; c0 -= kCbAhead) {
#pragma unroll
        for (int q = 0; q < kCbAhead; ++q)
            if (c0 - q >= 0) cb_bwd_step<T, DK>(a, L, stg[q], c0 - q, bh, rb, col0, wave, d);
    }
    if (a.dS0) {
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int tt = wave * TPW + u;
            if (tt < RT) {
#pragma unroll
                for (int v = 0; v < kCbCT; ++v)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        a.dS0[(bh * DK + 16 * tt + 4 * g4 + i) * a.DV + col0 + 16 * v + j] = d[u][v][i];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Token gradients of one chunk, or of a chunk pair.
// ---------------------------------------------------------------------------
template <int DK, int DV> struct alignas(16) CbGradLds {
    static constexpr int LK = DK + 4, LV = DV + 4, LS = kCB + 4;
    float bm[kCB][LK];                           // bm = b - m
    float m[DK], bcm[DK], rs[DK];                // m, b_C - m, rowsum(S * dN)
    float rs0[DK];                               // rowsum(S * dN) of a pair's first chunk
    // dO, U, dW of a chunk; of a pair's second chunk when both are held
    float dO[kCB][LV], U[kCB][LV], dW[kCB][LV];
    // U, dO, dW of a pair's first chunk
    float U0[kCB][LV], dO1[kCB][LV], dW1[kCB][LV];
    float X[kCB][LS], At[kCB][LS], dX[kCB][LS], Y[kCB][LS], dP[kCB][LS], dAt[kCB][LS];
    float bet[kCB];
};

// Per-lane operands that turn a stored neighbour state into this chunk's:
// the K^ rows and e^{b_C} of the previous chunk (the state entering this
// chunk is Diag(e^{b_C}) S + K^^T U of the previous one), or the Q~, K~ rows
// and e^{b_C} of the next chunk (the gradient leaving this chunk is
// Diag(e^{b_C}) dN + Q~^T dO - K~^T dW of the next one).
template <int NT> struct CbNeighbour {
    floatx4 r1[NT], r2[NT];
    float e[NT];
};

// Waves of a gradient workgroup: one 16-channel tile each at dk = 128 (eight
// waves), four otherwise.
template <int DK> __host__ __device__ constexpr int cb_grad_waves() { return DK >= 128 ? 8 : 4; }
template <int DK> __host__ __device__ constexpr int cb_grad_tiles() {
    return (DK / 16 + cb_grad_waves<DK>() - 1) / cb_grad_waves<DK>();
}

// One chunk's place: chain row base, first token, valid tokens, workspace unit.
struct CbChunk {
    int64_t rb, t0, unit;
    int n;
};
__device__ __forceinline__ CbChunk cb_chunk(const CbArgs &a, int64_t bh, int c) {
    CbChunk k;
    k.rb = cb_rowbase(a, bh);
    k.t0 = (int64_t)c * kCB;
    k.n = (int)(a.T - k.t0 < kCB ? a.T - k.t0 : kCB);
    k.unit = bh * a.nc + c;
    return k;
}

// q, k of this lane's tokens 4 g4 + i and channels 16 ct + j (step 4), zero
// past the end; loaded first so that the latency is hidden.
template <typename T, int DK>
__device__ __forceinline__ void cb_grad_qk(const CbArgs &a, const CbChunk &ck, int wave,
                                           float (&qin)[cb_grad_tiles<DK>()][4],
                                           float (&kin)[cb_grad_tiles<DK>()][4]) {
    constexpr int RT = DK / 16, NW = cb_grad_waves<DK>(), NT = cb_grad_tiles<DK>();
    const int lane = threadIdx.x & 63, j = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        const int ch = 16 * (wave + NW * u < RT ? wave + NW * u : 0) + j;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g4 + i, rr = r < ck.n ? r : ck.n - 1;
            const int64_t off = (ck.rb + (ck.t0 + rr) * a.H) * DK + ch;
            qin[u][i] = cb_ld<T>(a.q, off);
            kin[u][i] = cb_ld<T>(a.k, off);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qin[u][i] = 4 * g4 + i < ck.n ? qin[u][i] : 0.f;
            kin[u][i] = 4 * g4 + i < ck.n ? kin[u][i] : 0.f;
        }
    }
}

// Step 1, a chunk's inputs in LDS: with `decay` the log-decays (bm, m,
// b_C - m); X, At and beta; dO into `dO` when given.
template <typename T, int DK, int DV>
__device__ __forceinline__ void cb_grad_inputs(const CbArgs &a, CbGradLds<DK, DV> &L,
                                               const CbChunk &ck, bool decay,
                                               float (*dO)[CbGradLds<DK, DV>::LV]) {
    constexpr int NW = cb_grad_waves<DK>();
    const int tid = threadIdx.x;
    if (decay && tid < DK) {
        float gv[kCB], b[kCB];
        cb_load16<float>(a.g, ck.rb, ck.t0, ck.n, a.H, DK, tid, gv);
        cb_cumsum(gv, b);
        const float m = b[7];
        L.m[tid] = m;
        L.bcm[tid] = b[kCB - 1] - m;
#pragma unroll
        for (int r = 0; r < kCB; ++r) L.bm[r][tid] = b[r] - m;
    }
    if (dO) {
        for (int e = tid; e < kCB * DV; e += NW * 64) {
            const int r = e / DV, cc = e % DV;
            const int rr = r < ck.n ? r : ck.n - 1;
            const float ov = cb_ld<T>(a.dout, (ck.rb + (ck.t0 + rr) * a.H) * DV + cc);
            dO[r][cc] = r < ck.n ? ov : 0.f;
        }
    }
    const float *mc = a.mat + ck.unit * kCbMat;
    if (tid < kCB * kCB) {
        const int r = tid >> 4, cc = tid & 15;
        L.X[r][cc] = mc[r * kCB + cc];
        L.At[r][cc] = mc[2 * kCB * kCB + r * kCB + cc];
    }
    if (tid < kCB) L.bet[tid] = (tid < ck.n) ? cb_ld<T>(a.beta, ck.rb + (ck.t0 + tid) * a.H) : 0.f;
}

// Step 2, U = X Diag(beta) W and dW = Diag(beta) X^T dU into `U` and `dW`,
// column tiles over waves; dv = dW.
template <typename T, int DK, int DV>
__device__ __forceinline__ void cb_grad_u_dw(const CbArgs &a, CbGradLds<DK, DV> &L,
                                             const CbChunk &ck, int wave,
                                             float (*U)[CbGradLds<DK, DV>::LV],
                                             float (*dW)[CbGradLds<DK, DV>::LV]) {
    constexpr int CT = DV / 16, NW = cb_grad_waves<DK>();
    const int lane = threadIdx.x & 63, j = lane & 15, g4 = lane >> 4;
    const float *wc = a.w + ck.unit * kCB * DV;    // W, dU of the chunk: [16][DV]
    const float *duc = a.du + ck.unit * kCB * DV;
    for (int ct = wave; ct < CT; ct += NW) {
        const int cc = 16 * ct + j;
        floatx4 u4 = {0, 0, 0, 0}, w4 = {0, 0, 0, 0};
        const floatx4 xr = *reinterpret_cast<const floatx4 *>(&L.X[j][4 * g4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int s = 4 * g4 + i;
            u4 = mfma1(xr[i], L.bet[s] * wc[s * DV + cc], u4);
            w4 = mfma1(L.X[s][j], duc[s * DV + cc], w4);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g4 + i;
            w4[i] *= L.bet[r];
            U[r][cc] = u4[i];
            dW[r][cc] = w4[i];
            if (r < ck.n) a.dv[(ck.rb + (ck.t0 + r) * a.H) * DV + cc] = w4[i];
        }
    }
}

// Step 3a, the 16x16 chunk matrices (waves 0 and 1), with the chunk's dO and
// U from `dO`, `U`.
template <typename T, int DK, int DV>
__device__ __forceinline__ void cb_grad_mats(const CbArgs &a, CbGradLds<DK, DV> &L,
                                             const CbChunk &ck, int wave,
                                             const float (*dO)[CbGradLds<DK, DV>::LV],
                                             const float (*U)[CbGradLds<DK, DV>::LV]) {
    using Lds = CbGradLds<DK, DV>;
    const int lane = threadIdx.x & 63, j = lane & 15, g4 = lane >> 4;
    const float *wc = a.w + ck.unit * kCB * DV;
    const float *duc = a.du + ck.unit * kCB * DV;
    if (wave == 0) {
        floatx4 dT = {0, 0, 0, 0};                // dT[r][s] = dU_r . W_s
#pragma unroll
        for (int kb = 0; kb < DV / 16; ++kb) {
            const floatx4 x4 = ld4(duc + j * DV + 16 * kb + 4 * g4);
            const floatx4 y4 = ld4(wc + j * DV + 16 * kb + 4 * g4);
#pragma unroll
            for (int i = 0; i < 4; ++i) dT = mfma1(x4[i], y4[i], dT);
        }
        float dbT = 0.f;                          // sum_r X_rs dT_rs, column s = j
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g4 + i;
            dbT += L.X[r][j] * dT[i];
            L.dX[r][j] = dT[i] * L.bet[j];
        }
        dbT += __shfl_xor(dbT, 16);
        dbT += __shfl_xor(dbT, 32);
        // Y = dX X^T, then dA = -(X^T Y) below the diagonal
        floatx4 Yt = {0, 0, 0, 0};
        tile_mma<float>(Yt, &L.dX[0][0], Lds::LS, &L.X[0][0], Lds::LS, kCB, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) L.Y[4 * g4 + i][j] = Yt[i];
        floatx4 Z = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) Z = mfma1(L.X[4 * g4 + i][j], L.Y[4 * g4 + i][j], Z);
        float dbA[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g4 + i;
            const float dA = (j < r) ? -Z[i] : 0.f;
            dbA[i] = dA * L.At[r][j];
            L.dAt[r][j] = L.bet[r] * dA;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dbA[i] += __shfl_xor(dbA[i], 1);
            dbA[i] += __shfl_xor(dbA[i], 2);
            dbA[i] += __shfl_xor(dbA[i], 4);
            dbA[i] += __shfl_xor(dbA[i], 8);
        }
        // row r = 4 g4 + i sits in lane j = r of its column (dbT) and in lanes 16 g4.. (dbA)
        const float rowpart = dbA[0] * (j % 4 == 0) + dbA[1] * (j % 4 == 1) + dbA[2] * (j % 4 == 2) +
                              dbA[3] * (j % 4 == 3);
        // lane 16 g4 + j holds dbA of row 4 g4 + (j % 4); gather row r = lane (< 16)
        const float dbA_r = __shfl(rowpart, 16 * (lane >> 2) + (lane & 3));
        if (lane < kCB && lane < ck.n) a.dbeta[(ck.rb + (ck.t0 + lane) * a.H)] = dbT + dbA_r;
    } else if (wave == 1) {
        floatx4 dp = {0, 0, 0, 0};
        tile_mma<float>(dp, &dO[0][0], Lds::LV, &U[0][0], Lds::LV, DV, lane);  // dO_r . U_s
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g4 + i;
            L.dP[r][j] = (j <= r) ? dp[i] : 0.f;
        }
    }
}

// Step 3b's products of one 16x16 block of the state S and of the gradient dN
// (the chunk's own): dQ~ += dO S^T, dK~ += dW S^T, dK^ += U dN^T and the row
// sums of S * dN.
template <int DV>
__device__ __forceinline__ void cb_grad_block(const float (*dO)[DV + 4], const float (*dW)[DV + 4],
                                              const float (*U)[DV + 4], int k0, floatx4 sv,
                                              floatx4 nv, floatx4 &dQt, floatx4 &dKt,
                                              floatx4 &dKh, float &rsum) {
    const int lane = threadIdx.x & 63, j = lane & 15, g4 = lane >> 4;
    const floatx4 o4 = ld4(&dO[j][k0 + 4 * g4]);
    const floatx4 w4 = ld4(&dW[j][k0 + 4 * g4]);
    const floatx4 u4 = ld4(&U[j][k0 + 4 * g4]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        dQt = mfma1(o4[i], sv[i], dQt);
        dKt = mfma1(w4[i], sv[i], dKt);
        dKh = mfma1(u4[i], nv[i], dKh);
        rsum += sv[i] * nv[i];
    }
}

// Step 4, the pair terms and the token gradients of this wave's channel
// tiles, from step 3b's products and row sums `rs`.
template <typename T, int DK, int DV>
__device__ __forceinline__ void cb_grad_tokens(const CbArgs &a, CbGradLds<DK, DV> &L,
                                               const CbChunk &ck, int wave,
                                               const float (&qin)[cb_grad_tiles<DK>()][4],
                                               const float (&kin)[cb_grad_tiles<DK>()][4],
                                               const floatx4 (&dQt)[cb_grad_tiles<DK>()],
                                               const floatx4 (&dKt)[cb_grad_tiles<DK>()],
                                               const floatx4 (&dKh)[cb_grad_tiles<DK>()],
                                               const float *rs) {
    constexpr int RT = DK / 16, NW = cb_grad_waves<DK>(), NT = cb_grad_tiles<DK>();
    const int lane = threadIdx.x & 63, j = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        const int ct = wave + NW * u;
        if (ct >= RT) continue;
        const int ch = 16 * ct + j;
        const float *qv = qin[u], *kv = kin[u];
        floatx4 dQp = {0, 0, 0, 0}, dKp = {0, 0, 0, 0}, dKpp = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int s = 4 * g4 + i;
            const float bms = L.bm[s][ch], ks = kv[i], qs = qv[i];
            const float e = exp_hw(bms), ei = exp_hw(-bms);
            const float kpp = ks * ei, kp = ks * e, qp = qs * e;
            dQp = mfma1(L.dP[j][s], kpp, dQp);
            dKp = mfma1(L.dAt[j][s], kpp, dKp);
            dKpp = mfma1(L.dAt[s][j], kp, dKpp);
            dKpp = mfma1(L.dP[s][j], qp, dKpp);
        }
        const float m = L.m[ch], bcm = L.bcm[ch];
        float db[4], khk = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g4 + i;
            const float bmr = L.bm[r][ch], qr = qv[i], kr = kv[i];
            const float e_bm = exp_hw(bmr), e_mb = exp_hw(-bmr);
            const float e_b = exp_hw(bmr + m), e_cb = exp_hw(bcm - bmr);
            const float dq = dQt[u][i] * e_b + dQp[i] * e_bm;
            const float dk = -dKt[u][i] * e_b + dKh[u][i] * e_cb + dKp[i] * e_bm + dKpp[i] * e_mb;
            const float kh = dKh[u][i] * kr * e_cb;
            db[i] = dQt[u][i] * qr * e_b - dKt[u][i] * kr * e_b - kh + dQp[i] * qr * e_bm +
                    dKp[i] * kr * e_bm - dKpp[i] * kr * e_mb;
            khk += kh;
            if (r < ck.n) {
                const int64_t row = (ck.rb + (ck.t0 + r) * a.H);
                a.dq[row * DK + ch] = dq;
                a.dk[row * DK + ch] = dk;
            }
        }
        // suffix sums over the chunk's tokens (rows 4 g4 + i live in lane group g4)
        khk += __shfl_xor(khk, 16);
        khk += __shfl_xor(khk, 32);
        const float extra = khk + exp_hw(bcm + m) * rs[ch];
        db[2] += db[3];
        db[1] += db[2];
        db[0] += db[1];
        const float tot = db[0];
        const float t1 = __shfl(tot, j + 16), t2 = __shfl(tot, j + 32), t3 = __shfl(tot, j + 48);
        const float later = (g4 < 1 ? t1 : 0.f) + (g4 < 2 ? t2 : 0.f) + (g4 < 3 ? t3 : 0.f);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g4 + i;
            if (r < ck.n) a.dg[(ck.rb + (ck.t0 + r) * a.H) * DK + ch] = db[i] + later + extra;
        }
    }
}

// Token gradients of a chain's last chunk when it has no pair partner: the
// state entering it is read at sglob and the gradient leaving it at nglob.
template <typename T, int DK, int DV>
__device__ __forceinline__ void cb_grad_single(const CbArgs &a, CbGradLds<DK, DV> &L, int64_t bh,
                                               int c, int wave, const float *sglob,
                                               const float *nglob) {
    constexpr int RT = DK / 16, KB = DV / 16;
    constexpr int NW = cb_grad_waves<DK>(), NT = cb_grad_tiles<DK>();
    const int lane = threadIdx.x & 63, j = lane & 15, g4 = lane >> 4;
    const CbChunk ck = cb_chunk(a, bh, c);
    float qin[NT][4], kin[NT][4];
    cb_grad_qk<T, DK>(a, ck, wave, qin, kin);
    lds_barrier();
    cb_grad_inputs<T, DK, DV>(a, L, ck, true, L.dO);
    lds_barrier();
    cb_grad_u_dw<T, DK, DV>(a, L, ck, wave, L.U, L.dW);
    lds_barrier();
    cb_grad_mats<T, DK, DV>(a, L, ck, wave, L.dO, L.U);
    // 3b. the state products, channel tiles over waves
    floatx4 dQt[NT], dKt[NT], dKh[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        const int ct = wave + NW * u;
        dQt[u] = dKt[u] = dKh[u] = floatx4{0, 0, 0, 0};
        if (ct < RT) {
            const int cr = 16 * ct + j;
            float rsum = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int k0 = 16 * kb;
                const floatx4 sv = ld4(sglob + (int64_t)cr * DV + k0 + 4 * g4);
                const floatx4 nv = ld4(nglob + (int64_t)cr * DV + k0 + 4 * g4);
                cb_grad_block<DV>(L.dO, L.dW, L.U, k0, sv, nv, dQt[u], dKt[u], dKh[u], rsum);
            }
            rsum += __shfl_xor(rsum, 16);
            rsum += __shfl_xor(rsum, 32);
            if (g4 == 0) L.rs[cr] = rsum;
        }
    }
    lds_barrier();
    cb_grad_tokens<T, DK, DV>(a, L, ck, wave, qin, kin, dQt, dKt, dKh, L.rs);
}

// Token gradients of the chunk pair (c0, c1) = (2p, 2p+1) of one chain.  The
// passes stored the state entering c0 (sglob) and the gradient leaving c1
// (nglob); c1's entering state is formed from the first, c0's leaving
// gradient from the second, one 16x16 block at a time where the products
// need it.  Both chunks' products run in one sweep over the two stored
// blocks, so each is read from memory once.
template <typename T, int DK, int DV>
__device__ __forceinline__ void cb_grad_pair(const CbArgs &a, CbGradLds<DK, DV> &L, int64_t bh,
                                             int c0, int wave, const float *sglob,
                                             const float *nglob) {
    constexpr int RT = DK / 16, KB = DV / 16;
    constexpr int NW = cb_grad_waves<DK>(), NT = cb_grad_tiles<DK>();
    const int lane = threadIdx.x & 63, j = lane & 15, g4 = lane >> 4;
    const CbChunk k0c = cb_chunk(a, bh, c0), k1c = cb_chunk(a, bh, c0 + 1);
    // c0's U, dW (and its dv) and dO, held for the whole pair
    cb_grad_inputs<T, DK, DV>(a, L, k0c, false, L.dO1);
    lds_barrier();
    cb_grad_u_dw<T, DK, DV>(a, L, k0c, wave, L.U0, L.dW1);
    // ---- c1: inputs, U and dW, chunk matrices
    lds_barrier();                               // the steps above are done with X, beta
    cb_grad_inputs<T, DK, DV>(a, L, k1c, true, L.dO);
    lds_barrier();
    cb_grad_u_dw<T, DK, DV>(a, L, k1c, wave, L.U, L.dW);
    // the K^ rows and e^{b_C} of c0 (c1's entering state), the Q~, K~ rows
    // and e^{b_C} of c1 (c0's leaving gradient), requested before the barrier
    CbNeighbour<NT> nbs, nbn;
    {
        const float *op0 = a.ops + k0c.unit * cb_ops_floats(DK);
        const float *op1 = a.ops + k1c.unit * cb_ops_floats(DK);
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            const int ch = 16 * (wave + NW * u < RT ? wave + NW * u : 0) + j;
            nbs.r1[u] = ld4(op0 + kOpKhT * DK + ch * kCB + 4 * g4);   // K^[4 g4 + i][ch]
            nbs.e[u] = op0[kOpEbc * DK + ch];
            nbn.r1[u] = ld4(op1 + kOpQtT * DK + ch * kCB + 4 * g4);   // Q~[4 g4 + i][ch]
            nbn.r2[u] = ld4(op1 + kOpKtT * DK + ch * kCB + 4 * g4);   // K~[4 g4 + i][ch]
            nbn.e[u] = op1[kOpEbc * DK + ch];
        }
    }
    lds_barrier();
    cb_grad_mats<T, DK, DV>(a, L, k1c, wave, L.dO, L.U);
    // ---- 3b of both chunks, channel tiles over waves
    floatx4 dQt1[NT], dKt1[NT], dKh1[NT], dQt0[NT], dKt0[NT], dKh0[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        const int ct = wave + NW * u;
        dQt1[u] = dKt1[u] = dKh1[u] = dQt0[u] = dKt0[u] = dKh0[u] = floatx4{0, 0, 0, 0};
        if (ct < RT) {
            const int cr = 16 * ct + j;
            float rsum1 = 0.f, rsum0 = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int k0 = 16 * kb;
                const floatx4 sv = ld4(sglob + (int64_t)cr * DV + k0 + 4 * g4);
                const floatx4 nv = ld4(nglob + (int64_t)cr * DV + k0 + 4 * g4);
                // c1: the state entering it, Diag(e^{b_C}) S + K^^T U of c0
                // (transposed form: rows of the block are value columns,
                // columns key channels, as sv is laid out)
                floatx4 sv1 = sv * nbs.e[u];
#pragma unroll
                for (int i = 0; i < 4; ++i) sv1 = mfma1(L.U0[4 * g4 + i][k0 + j], nbs.r1[u][i], sv1);
                cb_grad_block<DV>(L.dO, L.dW, L.U, k0, sv1, nv, dQt1[u], dKt1[u], dKh1[u], rsum1);
                // c0: the gradient leaving it, Diag(e^{b_C}) dN + Q~^T dO - K~^T dW of c1
                floatx4 nv0 = nv * nbn.e[u];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    nv0 = mfma1(L.dO[4 * g4 + i][k0 + j], nbn.r1[u][i], nv0);
                    nv0 = mfma1(-L.dW[4 * g4 + i][k0 + j], nbn.r2[u][i], nv0);
                }
                cb_grad_block<DV>(L.dO1, L.dW1, L.U0, k0, sv, nv0, dQt0[u], dKt0[u], dKh0[u], rsum0);
            }
            rsum1 += __shfl_xor(rsum1, 16);
            rsum1 += __shfl_xor(rsum1, 32);
            rsum0 += __shfl_xor(rsum0, 16);
            rsum0 += __shfl_xor(rsum0, 32);
            if (g4 == 0) {
                L.rs[cr] = rsum1;
                L.rs0[cr] = rsum0;
            }
        }
    }
    float qin[NT][4], kin[NT][4];
    cb_grad_qk<T, DK>(a, k1c, wave, qin, kin);
    lds_barrier();
    cb_grad_tokens<T, DK, DV>(a, L, k1c, wave, qin, kin, dQt1, dKt1, dKh1, L.rs);
    // ---- c0: inputs but dO (held since the start), chunk matrices, tokens
    cb_grad_qk<T, DK>(a, k0c, wave, qin, kin);
    lds_barrier();                               // c1's tokens are done with the chunk arrays
    cb_grad_inputs<T, DK, DV>(a, L, k0c, true, nullptr);
    lds_barrier();
    cb_grad_mats<T, DK, DV>(a, L, k0c, wave, L.dO1, L.U0);
    lds_barrier();
    cb_grad_tokens<T, DK, DV>(a, L, k0c, wave, qin, kin, dQt0, dKt0, dKh0, L.rs0);
}

// Token gradients of the chunk pair (2p, 2p+1) of one chain, or of the last
// chunk alone when the chain's chunk count is odd.  The passes stored the
// state entering chunk 2p and the gradient leaving chunk 2p+1 (or 2p when it
// is the last chunk).
template <typename T, int DK, int DV>
__global__ __launch_bounds__(cb_grad_waves<DK>() * 64) void cb_grad_kernel(CbArgs a) {
    using Lds = CbGradLds<DK, DV>;
    __shared__ Lds L;
    const int64_t pair = blockIdx.x;
    const int64_t bh = pair / a.np;
    const int c0 = 2 * (int)(pair % a.np);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float *stp = a.st + pair * DK * DV;
    const float *dnp = a.dn + pair * DK * DV;
    if (c0 + 1 >= a.nc) cb_grad_single<T, DK, DV>(a, L, bh, c0, wave, stp, dnp);
    else cb_grad_pair<T, DK, DV>(a, L, bh, c0, wave, stp, dnp);
}

// Workspace of one launch over T tokens: the snapshots of even chunks' states
// and of odd chunks' gradients, X/P/At, W and dU per chunk, decayed operands.
static size_t cbwd_segment_bytes(int64_t B, int64_t T, int64_t H, int dk, int dv) {
    const int64_t nbh = B * H, nc = (T + kCB - 1) / kCB, np = (nc + 1) / 2;
    auto r256 = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t st = r256((size_t)nbh * np * dk * dv * sizeof(float));
    const size_t mat = r256((size_t)nbh * nc * kCbMat * sizeof(float));
    const size_t wv = r256((size_t)nbh * nc * kCB * dv * sizeof(float));
    const size_t ops = r256((size_t)nbh * nc * cb_ops_floats(dk) * sizeof(float));
    return 2 * st + mat + 2 * wv + ops;
}

size_t cbwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int dk, int dv) {
    return cbwd_segment_bytes(B, T, H, dk, dv);
}

// Segments of seg tokens (a multiple of 32, so every segment starts a chunk
// pair): one launch's workspace for a segment, plus the states entering
// segments 1 .. n-1 and two gradient carries, each [B*H, dk, dv] fp32.
size_t cbwd_workspace_bytes_seg(int64_t B, int64_t T, int64_t H, int dk, int dv, int64_t seg) {
    if (seg <= 0 || seg >= T) return cbwd_segment_bytes(B, T, H, dk, dv);
    const int64_t nseg = (T + seg - 1) / seg;
    const size_t state = (size_t)B * H * dk * dv * sizeof(float);
    return cbwd_segment_bytes(B, seg, H, dk, dv) + (size_t)(nseg - 1 + 2) * state;
}

// As a function of the segment length the workspace is convex: the segment's
// buffers grow with it and the entering states shrink with it.  The smallest
// lies near sqrt(state bytes x T / segment bytes per token); lengths are
// multiples of 32 tokens.
static int64_t cbwd_min_units(int64_t B, int64_t T, int64_t H, int dk, int dv) {
    const int64_t umax = (T - 1) / 32;
    if (umax < 1) return 1;
    const double per_tok = (double)cbwd_segment_bytes(B, 32 * umax, H, dk, dv) / (32.0 * umax);
    const double state = (double)B * H * dk * dv * sizeof(float);
    int64_t u0 = (int64_t)(sqrt(state * (double)T / per_tok) / 32.0);
    int64_t best = 1;
    size_t best_b = SIZE_MAX;
    for (int64_t u = u0 - 4; u <= u0 + 4; ++u) {
        if (u < 1 || u > umax) continue;
        const size_t b = cbwd_workspace_bytes_seg(B, T, H, dk, dv, 32 * u);
        if (b < best_b) { best_b = b; best = u; }
    }
    return best;
}

size_t cbwd_min_workspace_bytes(int64_t B, int64_t T, int64_t H, int dk, int dv) {
    const size_t whole = cbwd_segment_bytes(B, T, H, dk, dv);
    if (T <= 32) return whole;
    const size_t seg = cbwd_workspace_bytes_seg(B, T, H, dk, dv, 32 * cbwd_min_units(B, T, H, dk, dv));
    return seg < whole ? seg : whole;
}

// The longest segment (a multiple of 32 tokens, or the whole sequence) whose
// workspace fits in `bytes`; 0 when none does.  Above the smallest point the
// workspace grows with the length, so a binary search there finds it.
int64_t cbwd_segment_tokens(int64_t B, int64_t T, int64_t H, int dk, int dv, size_t bytes) {
    if (cbwd_segment_bytes(B, T, H, dk, dv) <= bytes) return T;
    if (T <= 32) return 0;
    int64_t lo = cbwd_min_units(B, T, H, dk, dv), hi = (T - 1) / 32;
    if (cbwd_workspace_bytes_seg(B, T, H, dk, dv, 32 * lo) > bytes) return 0;
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) / 2;
        if (cbwd_workspace_bytes_seg(B, T, H, dk, dv, 32 * mid) <= bytes) lo = mid;
        else hi = mid - 1;
    }
    return 32 * lo;
}

template <typename T, int DK>
static hipError_t cb_inst(CbArgs a, int64_t nbh, hipStream_t s) {
    hipLaunchKernelGGL((cb_prep_kernel<T, DK>), dim3((unsigned)(nbh * a.nc)), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((cb_fwd_kernel<T, DK>), dim3((unsigned)(nbh * a.nsl)), dim3(256), 0, s, a, nbh);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((cb_bwd_kernel<T, DK>), dim3((unsigned)(nbh * a.nsl)), dim3(256), 0, s, a, nbh);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 grid((unsigned)(nbh * a.np)), gblock(cb_grad_waves<DK>() * 64);
    switch (a.DV) {
    case 32: hipLaunchKernelGGL((cb_grad_kernel<T, DK, 32>), grid, gblock, 0, s, a); break;
    case 64: hipLaunchKernelGGL((cb_grad_kernel<T, DK, 64>), grid, gblock, 0, s, a); break;
    case 128: hipLaunchKernelGGL((cb_grad_kernel<T, DK, 128>), grid, gblock, 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

static void cb_layout(CbArgs &a, char *p, int64_t nbh, int64_t T, int dk, int dv) {
    const int64_t nc = (T + kCB - 1) / kCB, np = (nc + 1) / 2;
    auto r256 = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t st = r256((size_t)nbh * np * dk * dv * sizeof(float));
    const size_t mat = r256((size_t)nbh * nc * kCbMat * sizeof(float));
    const size_t wv = r256((size_t)nbh * nc * kCB * dv * sizeof(float));
    a.st = reinterpret_cast<float *>(p);
    a.dn = reinterpret_cast<float *>(p + st);
    a.mat = reinterpret_cast<float *>(p + 2 * st);
    a.w = reinterpret_cast<float *>(p + 2 * st + mat);
    a.du = reinterpret_cast<float *>(p + 2 * st + mat + wv);
    a.ops = reinterpret_cast<float *>(p + 2 * st + mat + 2 * wv);
    a.T = T; a.nc = (int)nc; a.np = (int)np;
}

template <typename T, int DK>
static hipError_t cb_fwd_only(CbArgs a, int64_t nbh, hipStream_t s) {
    hipLaunchKernelGGL((cb_prep_kernel<T, DK>), dim3((unsigned)(nbh * a.nc)), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((cb_fwd_kernel<T, DK>), dim3((unsigned)(nbh * a.nsl)), dim3(256), 0, s, a, nbh);
    return hipGetLastError();
}

static hipError_t cb_dispatch(const CbArgs &a, int64_t nbh, int dk, int is_bf16, bool fwd_only,
                              hipStream_t s) {
    switch (dk) {
    case 32:
        if (fwd_only) return is_bf16 ? cb_fwd_only<bf16, 32>(a, nbh, s) : cb_fwd_only<float, 32>(a, nbh, s);
        return is_bf16 ? cb_inst<bf16, 32>(a, nbh, s) : cb_inst<float, 32>(a, nbh, s);
    case 64:
        if (fwd_only) return is_bf16 ? cb_fwd_only<bf16, 64>(a, nbh, s) : cb_fwd_only<float, 64>(a, nbh, s);
        return is_bf16 ? cb_inst<bf16, 64>(a, nbh, s) : cb_inst<float, 64>(a, nbh, s);
    case 128:
        if (fwd_only) return is_bf16 ? cb_fwd_only<bf16, 128>(a, nbh, s) : cb_fwd_only<float, 128>(a, nbh, s);
        return is_bf16 ? cb_inst<bf16, 128>(a, nbh, s) : cb_inst<float, 128>(a, nbh, s);
    default: return hipErrorInvalidValue;
    }
}

// Chunked prefill in fp32 arithmetic for shapes the prefill kernels do not
// take (fp32 inputs at dk = 128): cb_prep_kernel forms X, P, At and the
// decayed operands of every 16-token chunk, then the forward state pass runs
// with outputs.  Workspace: those per-chunk buffers.
size_t cb_prefill_workspace_bytes(int64_t B, int64_t T, int64_t H, int dk) {
    const int64_t nbh = B * H, nc = (T + kCB - 1) / kCB;
    auto r256 = [](size_t x) { return (x + 255) / 256 * 256; };
    return r256((size_t)nbh * nc * kCbMat * sizeof(float)) +
           r256((size_t)nbh * nc * cb_ops_floats(dk) * sizeof(float));
}

template <typename T, int DK>
static hipError_t cb_prefill_inst(const CbArgs &a, int64_t nbh, hipStream_t s) {
    hipLaunchKernelGGL((cb_prep_kernel<T, DK>), dim3((unsigned)(nbh * a.nc)), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((cb_fwd_kernel<T, DK, true>), dim3((unsigned)(nbh * a.nsl)), dim3(256), 0, s,
                       a, nbh);
    return hipGetLastError();
}

hipError_t launch_chunk_fwd_cb(const void *q, const void *k, const void *v, const float *g,
                               const void *beta, const float *S0, float *ST, void *o, void *ws,
                               size_t ws_bytes, int64_t B, int64_t T, int64_t H, int dk, int dv,
                               int is_bf16, const int *slots, int64_t n_slots, hipStream_t s) {
    if (dv % kCbNS || dk != 128 || !ws || ws_bytes < cb_prefill_workspace_bytes(B, T, H, dk))
        return hipErrorInvalidValue;
    const int64_t nbh = B * H, nc = (T + kCB - 1) / kCB;
    if (nbh * nc > 0x7fffffffLL) return hipErrorInvalidValue;
    auto r256 = [](size_t x) { return (x + 255) / 256 * 256; };
    CbArgs a = {};
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.g = g;
    a.S0 = S0; a.sfinal = ST; a.o = o;
    a.slots = slots; a.n_slots = n_slots;
    char *p = static_cast<char *>(ws);
    a.mat = reinterpret_cast<float *>(p);
    a.ops = reinterpret_cast<float *>(p + r256((size_t)nbh * nc * kCbMat * sizeof(float)));
    a.T = T; a.tseq = T; a.toff = 0;
    a.H = (int)H; a.DV = dv; a.nsl = dv / kCbNS; a.nc = (int)nc; a.np = (int)((nc + 1) / 2);
    return is_bf16 ? cb_prefill_inst<bf16, 128>(a, nbh, s) : cb_prefill_inst<float, 128>(a, nbh, s);
}

// With a workspace for the whole sequence, one launch of each kernel.  With a
// smaller one, the sequence runs in segments of `seg` tokens (the longest
// that fit; every segment starts a 16-token chunk pair, so the chunks and the
// decay references are those of one pass): a forward sweep over segments
// 0 .. n-2 (prep and forward state pass) leaves the state entering every
// later segment, then the segments run in reverse, each a full backward from
// its entering state, with the gradient of its final state carried from the
// segment after it.  The forward pass is thus done twice; the workspace is
// bounded by a segment instead of the sequence.
hipError_t launch_chunk_bwd_chunked(const void *q, const void *k, const void *v, const float *g,
                                    const void *beta, const float *S0, const void *dout,
                                    const float *dST, float *dq, float *dk_, float *dv_, float *dg,
                                    float *dbeta, float *dS0, float *ws, size_t ws_bytes, int64_t B,
                                    int64_t T, int64_t H, int dk, int dv, int is_bf16, hipStream_t s) {
    if (dv % kCbNS || dk % 16) return hipErrorInvalidValue;
    const int64_t nbh = B * H;
    const int64_t seg = cbwd_segment_tokens(B, T, H, dk, dv, ws_bytes);
    if (seg <= 0) return hipErrorInvalidValue;
    if (nbh * ((seg + kCB - 1) / kCB) > 0x7fffffffLL) return hipErrorInvalidValue;
    CbArgs a;
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.dout = dout;
    a.g = g;
    a.dq = dq; a.dk = dk_; a.dv = dv_; a.dg = dg; a.dbeta = dbeta;
    a.H = (int)H; a.DV = dv; a.nsl = dv / kCbNS;
    a.tseq = T;
    a.sfinal = nullptr;
    char *p = reinterpret_cast<char *>(ws);
    if (seg >= T) {
        cb_layout(a, p, nbh, T, dk, dv);
        a.toff = 0; a.S0 = S0; a.dST = dST; a.dS0 = dS0;
        return cb_dispatch(a, nbh, dk, is_bf16, false, s);
    }
    const int64_t nseg = (T + seg - 1) / seg;
    const size_t state = (size_t)nbh * dk * dv;      // floats
    float *bound = reinterpret_cast<float *>(p);     // state entering segment i at bound[(i-1) state]
    float *carry = bound + (size_t)(nseg - 1) * state;
    char *segws = reinterpret_cast<char *>(carry + 2 * state);
    // forward sweep: the state entering segments 1 .. n-1
    for (int64_t i = 0; i + 1 < nseg; ++i) {
        cb_layout(a, segws, nbh, seg, dk, dv);
        a.toff = i * seg;
        a.S0 = i == 0 ? S0 : bound + (size_t)(i - 1) * state;
        a.sfinal = bound + (size_t)i * state;
        a.dST = nullptr; a.dS0 = nullptr;
        if (hipError_t e = cb_dispatch(a, nbh, dk, is_bf16, true, s)) return e;
    }
    a.sfinal = nullptr;
    // reverse sweep: each segment's gradients, the state gradient carried back
    for (int64_t i = nseg - 1; i >= 0; --i) {
        const int64_t len = i == nseg - 1 ? T - i * seg : seg;
        cb_layout(a, segws, nbh, len, dk, dv);
        a.toff = i * seg;
        a.S0 = i == 0 ? S0 : bound + (size_t)(i - 1) * state;
        a.dST = i == nseg - 1 ? dST : carry + (size_t)((i + 1) & 1) * state;
        a.dS0 = i == 0 ? dS0 : carry + (size_t)(i & 1) * state;
        if (hipError_t e = cb_dispatch(a, nbh, dk, is_bf16, false, s)) return e;
    }
    return hipSuccess;
}

}  // namespace kda
