// KDA chunkwise prefill: one fused kernel per (batch, head, dv-slice).
//
// Method ("Kimi K3 internal structure analysis", section "Sequence mixing: 3
// KDA layers per global MLA layer"): the per-token recurrence
//     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
//     o_t = S_t^T q_t,  alpha_t = exp(g_t),  g_t in [-5, 0],
// evaluated chunkwise.  The page states that the gate's floor keeps every
// 16-token tile's cumulative log-decay inside (-80, 0), within bf16/fp32
// range, so diagonal and off-diagonal causal tiles are all dense products;
// the chunk algebra itself is not on the pages and is derived here.
//
// Chunk algebra (chunk of C = 64 tokens, S the state entering it, b_r the
// running sum of g inside the chunk, all per key channel):
//     A_rs = beta_r sum_c k_rc k_sc e^{b_rc - b_sc}      (s < r)
//     P_rs = sum_c q_rc k_sc e^{b_rc - b_sc}             (s <= r)
//     T    = (I + A)^{-1} Diag(beta)                     (UT / WY form)
//     W    = T (K * e^b),   U' = T V,   U = U' - W S     (delta-rule writes)
//     O    = (Q * e^b) S + P U
//     S   <- Diag(e^{b_C}) S + (K * e^{b_C - b})^T U
// Decay factors are referenced to 16-token subtile boundaries so that every
// factor fed to a product lies in [e^-80, e^80] (the page's bound):
//     lam_r = running sum of g inside r's subtile (in [-80, 0]),
//     Lam_I = the subtile total.  For rows r in subtile I and columns s in J:
//       J == I : e^{lam_r} * e^{-lam_s}                     (<= 1 * <= e^80)
//       J <  I : e^{lam_r} * e^{Lam_J - lam_s} * e^{sum_{J<K<I} Lam_K}  (all <= 1)
//
// Data flow per chunk (all on chip, the fp32 state lives in MFMA accumulator
// registers across chunks, a bf16/fp32 copy of it in LDS as an operand):
//   A  prep:    g -> lam, Lam; decayed operand tiles into LDS
//   B  scores:  A and P on MFMA (20 tiles of 16x16)
//   C  inverse: (I + A)^-1 by 16x16 blocks (forward substitution on the
//               diagonal blocks, block substitution below), then T
//   D  W = T K~, U' = T V on MFMA
//   E  U = U' - W S
//   F  O = Q~ S + P U (to HBM), S <- e^{b_C} S + K^^T U
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

struct ChunkArgs {
    const void *q, *k, *v;
    const float *g;
    const void *beta;
    const float *S0;
    float *ST;
    void *o;
    int64_t T;
    int H, DV, nslice, nbh, xcd_map;
};

// LDS plan (byte offsets).  LDK: pitch of token rows with channels contiguous;
// LDT: pitch of channel rows with tokens contiguous; LDF: fp32 64x64 pitch.
template <typename T, int DK, int NV> struct ChunkLds {
    static constexpr int E = sizeof(T);
    static constexpr int PAD = 16 / E;
    static constexpr int LDK = DK + PAD;
    static constexpr int LDT = kChunk + PAD;
    static constexpr int LDF = kChunk + 4;
    static constexpr int LDY = 20;
    // region 1, phases A-B: decayed score operands
    static constexpr int QR = 0;
    static constexpr int KR = QR + 64 * LDK * E;
    static constexpr int KC = KR + 64 * LDK * E;           // 10 tiles of 16 rows
    static constexpr int R1_OPS = KC + 160 * LDK * E;
    // region 1, phases B-D: A, X = (I+A)^-1, block temporaries, P, T
    static constexpr int AF = 0;
    static constexpr int XF = AF + 64 * LDF * 4;
    static constexpr int YF = XF + 64 * LDF * 4;
    static constexpr int P = YF + 3 * 16 * LDY * 4;
    static constexpr int TT = P + 64 * LDT * E;
    static constexpr int R1_INV = TT + 64 * LDT * E;
    // region 1, phases D-F: -W and U^T (over A and X, which are dead by then)
    static constexpr int WN = 0;
    static constexpr int UT = WN + 64 * LDK * E;
    static constexpr int R1_W = UT + NV * LDT * E;
    static_assert(R1_W <= P, "-W / U^T must not overlap P and T");
    static constexpr int R1 = R1_OPS > R1_INV ? R1_OPS : R1_INV;
    // region 2: operands of the state pass, the state copy, small tables
    static constexpr int QT = R1;
    static constexpr int KTT = QT + 64 * LDK * E;
    static constexpr int KHT = KTT + DK * LDT * E;
    static constexpr int VT = KHT + DK * LDT * E;
    static constexpr int ST = VT + NV * LDT * E;
    static constexpr int LAM = ST + NV * LDK * E;
    static constexpr int EBC = LAM + 4 * DK * 4;
    static constexpr int BETA = EBC + DK * 4;
    static constexpr int TOTAL = BETA + 64 * 4;
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// k extent of the causal product for row block I, rounded to the MFMA k step
// (the blocks above the diagonal inside that extent hold zeros).
template <typename T> __device__ __forceinline__ int kround(int I) {
    constexpr int ks = Mma<T>::kStep;
    return ((16 * (I + 1) + ks - 1) / ks) * ks;
}

__device__ __forceinline__ void store16(bf16 *p, const float *x) {
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) { a[j] = (bf16)x[j]; b[j] = (bf16)x[8 + j]; }
    reinterpret_cast<bf16x8 *>(p)[0] = a;
    reinterpret_cast<bf16x8 *>(p)[1] = b;
}
__device__ __forceinline__ void store16(float *p, const float *x) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
        reinterpret_cast<floatx4 *>(p)[j] = floatx4{x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]};
}

template <typename T, int DK, int NV>
__global__ __launch_bounds__(256, 1) void chunk_fwd_kernel(ChunkArgs a) {
    using Lds = ChunkLds<T, DK, NV>;
    constexpr int LDK = Lds::LDK, LDT = Lds::LDT, LDF = Lds::LDF, LDY = Lds::LDY;
    constexpr int NITEM = (4 * DK + 255) / 256;     // (channel, subtile) items per thread
    constexpr int NU = NV / 16;                      // U / O tiles per wave
    constexpr int NSB = NV / 16;                     // state column blocks
    constexpr int NS = (DK / 16) * NSB / 4;          // state tiles per wave
    static_assert(NS >= 1 && (DK / 16) * NSB % 4 == 0, "state tiles");

    __shared__ __attribute__((aligned(16))) unsigned char smem[Lds::TOTAL];
    T *sQr = reinterpret_cast<T *>(smem + Lds::QR);
    T *sKr = reinterpret_cast<T *>(smem + Lds::KR);
    T *sKc = reinterpret_cast<T *>(smem + Lds::KC);
    float *sAf = reinterpret_cast<float *>(smem + Lds::AF);
    float *sXf = reinterpret_cast<float *>(smem + Lds::XF);
    float *sYf = reinterpret_cast<float *>(smem + Lds::YF);
    T *sP = reinterpret_cast<T *>(smem + Lds::P);
    T *sT = reinterpret_cast<T *>(smem + Lds::TT);
    T *sWn = reinterpret_cast<T *>(smem + Lds::WN);
    T *sUT = reinterpret_cast<T *>(smem + Lds::UT);
    T *sQt = reinterpret_cast<T *>(smem + Lds::QT);
    T *sKtT = reinterpret_cast<T *>(smem + Lds::KTT);
    T *sKhT = reinterpret_cast<T *>(smem + Lds::KHT);
    T *sVT = reinterpret_cast<T *>(smem + Lds::VT);
    T *sST = reinterpret_cast<T *>(smem + Lds::ST);
    float *sLam = reinterpret_cast<float *>(smem + Lds::LAM);
    float *sEbC = reinterpret_cast<float *>(smem + Lds::EBC);
    float *sBeta = reinterpret_cast<float *>(smem + Lds::BETA);

    const T *__restrict__ q = static_cast<const T *>(a.q);
    const T *__restrict__ k = static_cast<const T *>(a.k);
    const T *__restrict__ v = static_cast<const T *>(a.v);
    const T *__restrict__ beta = static_cast<const T *>(a.beta);
    const float *__restrict__ g = a.g;
    T *__restrict__ o = static_cast<T *>(a.o);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg4 = (lane >> 4) * 4;

    // Work item: (chain bh, dv slice).  With the XCD mapping, the slices of
    // one chain land on the same XCD (workgroups are dealt round-robin over
    // the 8 XCDs) and share its L2 for q, k, g.
    int bh, slice;
    {
        const int id = blockIdx.x;
        if (a.xcd_map) {
            const int x = id & 7, j = id >> 3;
            bh = (j / a.nslice) * 8 + x;
            slice = j % a.nslice;
        } else {
            bh = id / a.nslice;
            slice = id % a.nslice;
        }
    }
    const int H = a.H, DV = a.DV;
    const int b = bh / H, h = bh % H;
    const int64_t T_ = a.T;
    const int vcol0 = slice * NV;

    // ---- state: fp32 accumulator tiles owned by this wave ----------------
    floatx4 sacc[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int ti = wave + 4 * i, cb = ti / NSB, nb = ti % NSB;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = 16 * cb + lg4 + j, n = vcol0 + 16 * nb + lr;
            sacc[i][j] = a.S0 ? a.S0[((int64_t)bh * DK + c) * DV + n] : 0.0f;
        }
        store4(sST + (16 * nb + lr) * LDK + 16 * cb + lg4, sacc[i][0], sacc[i][1], sacc[i][2],
               sacc[i][3]);
    }

    const int64_t nchunk = (T_ + kChunk - 1) / kChunk;
    for (int64_t ch = 0; ch < nchunk; ++ch) {
        const int64_t t0 = ch * kChunk;
        const int L = (int)((T_ - t0) < kChunk ? (T_ - t0) : kChunk);
        const int64_t tok0 = ((int64_t)b * T_ + t0) * H + h;   // token t0 + r -> tok0 + r*H

        // ---- A1: running log-decay inside each 16-token subtile -----------
        float lam[NITEM][16], kx[NITEM][16], qx[NITEM][16];
#pragma unroll
        for (int it = 0; it < NITEM; ++it) {
            const int item = tid + 256 * it;
            if (item < 4 * DK) {
                const int c = item % DK, I = item / DK;
                float run = 0.0f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int tl = 16 * I + r;
                    float gv = 0.0f, kv = 0.0f, qv = 0.0f;
                    if (tl < L) {
                        const int64_t e = (tok0 + (int64_t)tl * H) * DK + c;
                        gv = g[e];
                        kv = to_f32(k[e]);
                        qv = to_f32(q[e]);
                    }
                    run += gv;
                    lam[it][r] = run;
                    kx[it][r] = kv;
                    qx[it][r] = qv;
                }
                sLam[I * DK + c] = run;
            }
        }
        if (tid < 64) sBeta[tid] = (tid < L) ? to_f32(beta[tok0 + (int64_t)tid * H]) : 0.0f;
        for (int item = tid; item < NV * 4; item += 256) {
            const int n = item % NV, I = item / NV;
            float vv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int tl = 16 * I + r;
                vv[r] = (tl < L) ? to_f32(v[(tok0 + (int64_t)tl * H) * DV + vcol0 + n]) : 0.0f;
            }
            store16(sVT + n * LDT + 16 * I, vv);
        }
        __syncthreads();

        // ---- A2: decayed operand tiles -----------------------------------
#pragma unroll
        for (int it = 0; it < NITEM; ++it) {
            const int item = tid + 256 * it;
            if (item < 4 * DK) {
                const int c = item % DK, I = item / DK;
                const float L0 = sLam[c], L1 = sLam[DK + c], L2 = sLam[2 * DK + c],
                            L3 = sLam[3 * DK + c];
                const float pre1 = L0, pre2 = L0 + L1, pre3 = L0 + L1 + L2, pre4 = pre3 + L3;
                const float preI = I == 0 ? 0.0f : I == 1 ? pre1 : I == 2 ? pre2 : pre3;
                const float LamI = I == 0 ? L0 : I == 1 ? L1 : I == 2 ? L2 : L3;
                const float preI1 = preI + LamI;        // b at the end of subtile I
                const float ePre = __expf(preI);        // e^{b before subtile I}   <= 1
                const float eNegLam = __expf(-LamI);    // e^{-Lam_I}              <= e^80
                const float eHat = __expf(pre4 - preI1); // e^{b_C - b_end(I)}     <= 1
                const float eOff1 = __expf(pre1 - preI1);   // only used for I2 > I
                const float eOff2 = __expf(pre2 - preI1);
                const float eOff3 = __expf(pre3 - preI1);
                if (I == 0) sEbC[c] = __expf(pre4);
                float kt[16], kh[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int s = 16 * I + r;
                    const float lr_ = lam[it][r];
                    const float R = __expf(lr_);            // e^{lam_r}           in [e^-80, 1]
                    const float Et = __expf(LamI - lr_);    // e^{Lam_I - lam_r}   in [e^-75, 1]
                    const float kv = kx[it][r], qv = qx[it][r];
                    sKr[s * LDK + c] = from_f32<T>(kv * R);
                    sQr[s * LDK + c] = from_f32<T>(qv * R);
                    // diagonal pair (I, I): column factor e^{-lam_s} = Et * e^{-Lam_I}
                    sKc[((I * (I + 1)) / 2 + I) * 16 * LDK + r * LDK + c] =
                        from_f32<T>(kv * (Et * eNegLam));
                    // off-diagonal pairs (I2, I), I2 > I
                    if (I < 1) sKc[(1 + I) * 16 * LDK + r * LDK + c] = from_f32<T>(kv * Et * eOff1);
                    if (I < 2) sKc[(3 + I) * 16 * LDK + r * LDK + c] = from_f32<T>(kv * Et * eOff2);
                    if (I < 3) sKc[(6 + I) * 16 * LDK + r * LDK + c] = from_f32<T>(kv * Et * eOff3);
                    const float eb = R * ePre;                  // e^{b_r}  <= 1
                    sQt[s * LDK + c] = from_f32<T>(qv * eb);
                    kt[r] = kv * eb;
                    kh[r] = kv * Et * eHat;                     // e^{b_C - b_r} <= 1
                }
                store16(sKtT + c * LDT + 16 * I, kt);
                store16(sKhT + c * LDT + 16 * I, kh);
            }
        }
        __syncthreads();

        // ---- B: A and P tiles (10 causal subtile pairs each) ---------------
        floatx4 sc[5];
#pragma unroll
        for (int u = 0; u < 5; ++u) {
            const int ti = wave + 4 * u, p = ti >> 1;
            const int I = p >= 6 ? 3 : p >= 3 ? 2 : p >= 1 ? 1 : 0;
            sc[u] = floatx4{0, 0, 0, 0};
            tile_mma<T>(sc[u], sKc + p * 16 * LDK, LDK, ((ti & 1) ? sQr : sKr) + 16 * I * LDK,
                        LDK, DK, lane);
        }
        __syncthreads();   // region 1 is rewritten below
#pragma unroll
        for (int u = 0; u < 5; ++u) {
            const int ti = wave + 4 * u, p = ti >> 1;
            const int I = p >= 6 ? 3 : p >= 3 ? 2 : p >= 1 ? 1 : 0;
            const int J = p - (I * (I + 1)) / 2;
            const bool isP = ti & 1;
            float val[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int s = lg4 + j;                  // column inside block J
                const bool keep = (J < I) || (isP ? (s <= lr) : (s < lr));
                val[j] = keep ? sc[u][j] : 0.0f;
            }
            const int r = 16 * I + lr;
            if (isP) {
                store4(sP + r * LDT + 16 * J + lg4, val[0], val[1], val[2], val[3]);
            } else {
                const float bt = sBeta[r];
                store4(sAf + r * LDF + 16 * J + lg4, bt * val[0], bt * val[1], bt * val[2],
                       bt * val[3]);
            }
        }
        // zero the blocks above the diagonal of P and T (read by the rounded-up
        // causal products)
        for (int e = tid; e < 6 * 64; e += 256) {
            const int blk = e >> 6, q4 = e & 63, rr = q4 >> 2, cc = (q4 & 3) * 4;
            const int I = blk < 3 ? 0 : blk < 5 ? 1 : 2;
            const int J = blk < 3 ? blk + 1 : blk < 5 ? blk - 1 : 3;
            store4(sP + (16 * I + rr) * LDT + 16 * J + cc, 0.f, 0.f, 0.f, 0.f);
            store4(sT + (16 * I + rr) * LDT + 16 * J + cc, 0.f, 0.f, 0.f, 0.f);
        }
        __syncthreads();

        // ---- C1: diagonal blocks of (I + A)^-1, forward substitution ----------
        if (wave == 0) {
            const int I = lane >> 4, jc = lane & 15;
            const float *Ab = sAf + 16 * I * LDF + 16 * I;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float acc = 0.0f;
#pragma unroll
                for (int m = 0; m < i; ++m) acc = fmaf(Ab[i * LDF + m], x[m], acc);
                x[i] = (i < jc) ? 0.0f : ((i == jc) ? 1.0f : -acc);
            }
            float *Xb = sXf + 16 * I * LDF + 16 * I;
#pragma unroll
            for (int i = 0; i < 16; ++i) Xb[i * LDF + jc] = x[i];
        }
        __syncthreads();

        // ---- C2: blocks below the diagonal, X_IJ = -X_II sum_K A_IK X_KJ ---------
#pragma unroll
        for (int d = 1; d < 4; ++d) {
            const int nblk = 4 - d;
            const int bi = tid >> 6, e = tid & 63, i = e >> 2, j4 = (e & 3) * 4;
            const int J = bi, I = J + d;
            if (bi < nblk) {
                floatx4 y = {0, 0, 0, 0};
                for (int K = J; K < I; ++K) {
#pragma unroll
                    for (int m = 0; m < 16; ++m) {
                        const float av = sAf[(16 * I + i) * LDF + 16 * K + m];
                        const floatx4 xv =
                            *reinterpret_cast<const floatx4 *>(sXf + (16 * K + m) * LDF + 16 * J + j4);
                        y += av * xv;
                    }
                }
                *reinterpret_cast<floatx4 *>(sYf + (bi * 16 + i) * LDY + j4) = y;
            }
            __syncthreads();
            if (bi < nblk) {
                floatx4 xn = {0, 0, 0, 0};
                for (int m = 0; m <= i; ++m) {
                    const float xa = sXf[(16 * I + i) * LDF + 16 * I + m];
                    const floatx4 yv = *reinterpret_cast<const floatx4 *>(sYf + (bi * 16 + m) * LDY + j4);
                    xn += xa * yv;
                }
                *reinterpret_cast<floatx4 *>(sXf + (16 * I + i) * LDF + 16 * J + j4) = -xn;
            }
            __syncthreads();
        }

        // ---- C3: T = X Diag(beta) on and below the diagonal blocks --------
        for (int e = tid; e < 64 * 16; e += 256) {
            const int r = e >> 4, s4 = (e & 15) * 4;
            if ((s4 >> 4) <= (r >> 4)) {
                const floatx4 xv = *reinterpret_cast<const floatx4 *>(sXf + r * LDF + s4);
                store4(sT + r * LDT + s4, xv[0] * sBeta[s4], xv[1] * sBeta[s4 + 1],
                       xv[2] * sBeta[s4 + 2], xv[3] * sBeta[s4 + 3]);
            }
        }
        __syncthreads();

        // ---- D: -W = -T K~ into LDS; U' = T V into registers ---------------
        for (int ti = wave; ti < DK / 4; ti += 4) {
            const int cb = ti >> 2, I = ti & 3;
            floatx4 acc = {0, 0, 0, 0};
            tile_mma<T>(acc, sKtT + 16 * cb * LDT, LDT, sT + 16 * I * LDT, LDT, kround<T>(I), lane);
            store4(sWn + (16 * I + lr) * LDK + 16 * cb + lg4, -acc[0], -acc[1], -acc[2], -acc[3]);
        }
        floatx4 uacc[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int ti = wave + 4 * u, Is = ti & 3, nb = ti >> 2;
            uacc[u] = floatx4{0, 0, 0, 0};
            tile_mma<T>(uacc[u], sT + 16 * Is * LDT, LDT, sVT + 16 * nb * LDT, LDT, kround<T>(Is),
                        lane);
        }
        __syncthreads();

        // ---- E: U = U' - W S, stored transposed (tokens contiguous) -----------
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int ti = wave + 4 * u, Is = ti & 3, nb = ti >> 2;
            tile_mma<T>(uacc[u], sWn + 16 * Is * LDK, LDK, sST + 16 * nb * LDK, LDK, DK, lane);
            store4(sUT + (16 * nb + lr) * LDT + 16 * Is + lg4, uacc[u][0], uacc[u][1], uacc[u][2],
                   uacc[u][3]);
        }
        __syncthreads();

        // ---- F: outputs, then the state update ------------------------------
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int ti = wave + 4 * u, Ir = ti & 3, nb = ti >> 2;
            floatx4 acc = {0, 0, 0, 0};
            tile_mma<T>(acc, sST + 16 * nb * LDK, LDK, sQt + 16 * Ir * LDK, LDK, DK, lane);
            tile_mma<T>(acc, sUT + 16 * nb * LDT, LDT, sP + 16 * Ir * LDT, LDT, kround<T>(Ir), lane);
            const int r = 16 * Ir + lr;
            if (r < L)
                store4(o + (tok0 + (int64_t)r * H) * DV + vcol0 + 16 * nb + lg4, acc[0], acc[1],
                       acc[2], acc[3]);
        }
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int ti = wave + 4 * i, cb = ti / NSB, nb = ti % NSB;
#pragma unroll
            for (int j = 0; j < 4; ++j) sacc[i][j] *= sEbC[16 * cb + lg4 + j];
            tile_mma<T>(sacc[i], sKhT + 16 * cb * LDT, LDT, sUT + 16 * nb * LDT, LDT, kChunk, lane);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int ti = wave + 4 * i, cb = ti / NSB, nb = ti % NSB;
            store4(sST + (16 * nb + lr) * LDK + 16 * cb + lg4, sacc[i][0], sacc[i][1], sacc[i][2],
                   sacc[i][3]);
        }
    }

    if (a.ST) {
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int ti = wave + 4 * i, cb = ti / NSB, nb = ti % NSB;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = 16 * cb + lg4 + j, n = vcol0 + 16 * nb + lr;
                a.ST[((int64_t)bh * DK + c) * DV + n] = sacc[i][j];
            }
        }
    }
}

// dv-slice width per workgroup for each (dtype, dk): the widest that fits LDS.
static int slice_width(int dk, int dv, int is_bf16) {
    int nv = is_bf16 ? 64 : 32;
    if (nv > dv) nv = dv;
    (void)dk;
    return nv;
}

bool chunk_fwd_supported(int dk, int dv, int is_bf16) {
    const bool dk_ok = is_bf16 ? (dk == 32 || dk == 64 || dk == 128) : (dk == 32 || dk == 64);
    return dk_ok && (dv == 32 || dv == 64 || dv == 128);
}

template <typename T, int DK, int NV>
static hipError_t launch_inst(const ChunkArgs &args, int nblocks, hipStream_t s) {
    hipLaunchKernelGGL((chunk_fwd_kernel<T, DK, NV>), dim3(nblocks), dim3(256), 0, s, args);
    return hipGetLastError();
}

hipError_t launch_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                            const void *beta, const float *S0, float *ST, void *o, int64_t B,
                            int64_t T, int64_t H, int dk, int dv, int is_bf16, hipStream_t s) {
    if (!chunk_fwd_supported(dk, dv, is_bf16)) return hipErrorInvalidValue;
    const int nv = slice_width(dk, dv, is_bf16);
    ChunkArgs args;
    args.q = q; args.k = k; args.v = v; args.g = g; args.beta = beta;
    args.S0 = S0; args.ST = ST; args.o = o;
    args.T = T; args.H = (int)H; args.DV = dv; args.nslice = dv / nv;
    args.nbh = (int)(B * H);
    args.xcd_map = (args.nbh % 8 == 0) ? 1 : 0;
    const int nblocks = args.nbh * args.nslice;
    if (is_bf16) {
        switch (dk * 1000 + nv) {
        case 32032: return launch_inst<bf16, 32, 32>(args, nblocks, s);
        case 32064: return launch_inst<bf16, 32, 64>(args, nblocks, s);
        case 64032: return launch_inst<bf16, 64, 32>(args, nblocks, s);
        case 64064: return launch_inst<bf16, 64, 64>(args, nblocks, s);
        case 128032: return launch_inst<bf16, 128, 32>(args, nblocks, s);
        case 128064: return launch_inst<bf16, 128, 64>(args, nblocks, s);
        default: return hipErrorInvalidValue;
        }
    }
    switch (dk * 1000 + nv) {
    case 32032: return launch_inst<float, 32, 32>(args, nblocks, s);
    case 64032: return launch_inst<float, 64, 32>(args, nblocks, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
