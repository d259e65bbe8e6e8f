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
//     X    = (I + A)^{-1}                               (UT / WY form)
//     W    = X (beta K e^b),  U' = X (beta V),  U = U' - W S   (delta-rule writes)
//     O    = (Q e^b) S + P U
//     S   <- Diag(e^{b_C}) S + (K e^{b_C - b})^T U
// Decay factors are referenced to 16-token subtile boundaries so that every
// factor fed to a product lies in [e^-80, e^80] (the page's bound):
//     lam_r = running sum of g inside r's subtile (in [-80, 0]),
//     Lam_I = the subtile total.  For rows r in subtile I and columns s in J:
//       J == I : e^{lam_r} * e^{-lam_s}                               (<= 1 * <= e^80)
//       J <  I : e^{lam_r} * e^{Lam_J - lam_s} * e^{sum_{J<K<I} Lam_K}   (all <= 1)
//
// Work per chunk (one workgroup of 4 waves; wave w owns subtile w in the
// intra-chunk stages and dv column block(s) w, w+4, .. in the state pass):
//   A  prep     raw q/k/v/g/beta (prefetched into registers one chunk ahead
//               with 8/16-byte loads) -> in-wave running sums -> decayed
//               operand tiles in LDS (beta folded into K and V rows)
//   B  scores   A and P, 20 16x16 tiles on MFMA; P kept as bf16 hi + lo
//   C  inverse  X = (I + A)^-1 on MFMA: diagonal 16x16 blocks by the product
//               (I+N)(I+N^2)(I+N^4)(I+N^8) with N = -A_II (A_II^16 = 0), the
//               blocks below by block substitution, one level per barrier
//   D  W, U'    on MFMA
//   E  state    per wave, no barrier: U = U' - W S (kept as bf16 hi + lo),
//               O = Q~ S + P U to HBM, S <- e^{b_C} S + K^^T U (fp32 state in
//               MFMA accumulator registers, a bf16 copy in LDS as an operand)
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

// Four consecutive elements of T in one register group.
template <typename T> struct Quad;
template <> struct Quad<bf16> { typedef bf16x4 type; };
template <> struct Quad<float> { typedef floatx4 type; };

__device__ __forceinline__ floatx4 to_f4(bf16x4 x) {
    return floatx4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}
__device__ __forceinline__ floatx4 to_f4(floatx4 x) { return x; }

// LDS plan (byte offsets).  LDK: pitch of token rows (channels contiguous);
// LDT: pitch of channel rows (tokens contiguous).
template <typename T, int DK, int NV> struct ChunkLds {
    static constexpr int E = sizeof(T);
    static constexpr int PAD = 16 / E;
    static constexpr int LDK = DK + PAD;
    static constexpr int LDT = kChunk + PAD;
    static constexpr int TILE64 = 64 * LDT * E;          // one [64][LDT] matrix
    static constexpr bool SPLIT = sizeof(T) == 2;        // bf16 keeps P and U as hi + lo
    // region 1, stages A-B: decayed score operands
    static constexpr int QR = 0;
    static constexpr int KR = QR + 64 * LDK * E;
    static constexpr int KC = KR + 64 * LDK * E;          // 10 tiles of 16 rows
    static constexpr int R1_OPS = KC + 160 * LDK * E;
    // region 1, stages B-E: P (hi, lo), X row- and column-major, A
    static constexpr int PH = 0;
    static constexpr int PL = PH + TILE64;
    static constexpr int XR = PL + (SPLIT ? TILE64 : 0);
    static constexpr int XC = XR + TILE64;
    static constexpr int AB = XC + TILE64;
    static constexpr int R1_INV = AB + TILE64;
    // stage D on: -W over XC and AB (dead by then); stage E: U^T hi over XR
    // (dead after stage D), U^T lo after AB
    static constexpr int WN = XC;
    static constexpr int UTH = XR;
    static constexpr int UTL = R1_INV;
    static_assert(64 * LDK * E <= 2 * TILE64, "-W must fit over X^c and A");
    static_assert(NV * LDT * E <= TILE64, "U^T hi must fit over X");
    static constexpr int R1_E = UTL + (SPLIT ? NV * LDT * E : 0);
    static constexpr int R1 = R1_OPS > R1_E ? R1_OPS : R1_E;
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

// ---------------------------------------------------------------------------
// 16x16x16 products in the accumulator ("L") layout: lane l holds
// M[4*(l/16) + j][l % 16] in element j.  mma16(L(X^T), L(Y)) = L(X Y).
// ---------------------------------------------------------------------------
__device__ __forceinline__ floatx4 mma16(bf16, floatx4 a, floatx4 b, floatx4 c) {
    bf16x4 ab = {(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3]};
    bf16x4 bb = {(bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ab, bb, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma16(float, floatx4 a, floatx4 b, floatx4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
}

// Four consecutive T values from LDS as fp32, and back.
__device__ __forceinline__ floatx4 lds_load4(const bf16 *p) {
    return to_f4(*reinterpret_cast<const bf16x4 *>(p));
}
__device__ __forceinline__ floatx4 lds_load4(const float *p) {
    return *reinterpret_cast<const floatx4 *>(p);
}
template <typename T> __device__ __forceinline__ void store4v(T *p, floatx4 x) {
    store4(p, x[0], x[1], x[2], x[3]);
}

// N consecutive values (channel-major rows: tokens contiguous).
template <int N> __device__ __forceinline__ void storeN(bf16 *p, const float *x) {
    if constexpr (N == 2) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<bf16x2 *>(p) = bf16x2{(bf16)x[0], (bf16)x[1]};
    } else {
#pragma unroll
        for (int i = 0; i < N; i += 4) store4(p + i, x[i], x[i + 1], x[i + 2], x[i + 3]);
    }
}
template <int N> __device__ __forceinline__ void storeN(float *p, const float *x) {
    if constexpr (N == 2) {
        typedef float floatx2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<floatx2 *>(p) = floatx2{x[0], x[1]};
    } else {
#pragma unroll
        for (int i = 0; i < N; i += 4) store4(p + i, x[i], x[i + 1], x[i + 2], x[i + 3]);
    }
}

// Order this wave's earlier LDS writes before its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T, int DK, int NV>
__global__ __launch_bounds__(256, 1) void chunk_fwd_kernel(ChunkArgs a) {
    using Lds = ChunkLds<T, DK, NV>;
    using T4 = typename Quad<T>::type;
    constexpr int LDK = Lds::LDK, LDT = Lds::LDT;
    constexpr bool kSplit = Lds::SPLIT;              // keep P and U as bf16 hi + lo
    // prep mapping: thread = (channel quad cq, token group tg); wave w <-> subtile w
    constexpr int NQ = DK / 4;                       // channel quads
    constexpr int TPT = DK / 16;                     // tokens per thread (8, 4, 2)
    constexpr int NVQ = NV / 4;                      // dv quads of the slice
    constexpr int TPV = NV / 16;                     // v tokens per thread
    constexpr int NSB = NV / 16;                     // state column blocks
    constexpr int NOWN = (NSB + 3) / 4;              // column blocks owned per wave
    constexpr int NCB = DK / 16;                     // state row blocks
    static_assert(256 == NQ * (64 / TPT) && 256 == NVQ * (64 / TPV), "prep mapping");

    __shared__ __attribute__((aligned(16))) unsigned char smem[Lds::TOTAL];
    T *sQr = reinterpret_cast<T *>(smem + Lds::QR);
    T *sKr = reinterpret_cast<T *>(smem + Lds::KR);
    T *sKc = reinterpret_cast<T *>(smem + Lds::KC);
    T *sPh = reinterpret_cast<T *>(smem + Lds::PH);
    T *sPl = reinterpret_cast<T *>(smem + Lds::PL);
    T *sXr = reinterpret_cast<T *>(smem + Lds::XR);
    T *sXc = reinterpret_cast<T *>(smem + Lds::XC);
    T *sA = reinterpret_cast<T *>(smem + Lds::AB);
    T *sWn = reinterpret_cast<T *>(smem + Lds::WN);
    T *sUh = reinterpret_cast<T *>(smem + Lds::UTH);
    T *sUl = reinterpret_cast<T *>(smem + Lds::UTL);
    T *sQt = reinterpret_cast<T *>(smem + Lds::QT);
    T *sKtT = reinterpret_cast<T *>(smem + Lds::KTT);
    T *sKhT = reinterpret_cast<T *>(smem + Lds::KHT);
    T *sVT = reinterpret_cast<T *>(smem + Lds::VT);
    T *sST = reinterpret_cast<T *>(smem + Lds::ST);
    float *sLam = reinterpret_cast<float *>(smem + Lds::LAM);
    float *sEbC = reinterpret_cast<float *>(smem + Lds::EBC);
    float *sBeta = reinterpret_cast<float *>(smem + Lds::BETA);

    const T *__restrict__ qp = static_cast<const T *>(a.q);
    const T *__restrict__ kp = static_cast<const T *>(a.k);
    const T *__restrict__ vp = static_cast<const T *>(a.v);
    const T *__restrict__ bp = static_cast<const T *>(a.beta);
    const float *__restrict__ gp = a.g;
    T *__restrict__ op = static_cast<T *>(a.o);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg4 = (lane >> 4) * 4;
    const int cq = tid % NQ, tg = tid / NQ, pos = lane / NQ;   // pos: rank inside the subtile
    const int vq = tid % NVQ, tv = tid / NVQ;

    // Work item (chain bh, dv slice).  With the XCD mapping the slices of one
    // chain land on one XCD (workgroups are dealt round-robin over 8 XCDs) and
    // share its L2 for q, k, g.
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
    const int64_t nchunk = (T_ + kChunk - 1) / kChunk;

    // ---- raw chunk inputs, prefetched one chunk ahead ---------------------
    floatx4 rg[TPT];
    T4 rk[TPT], rq[TPT], rv[TPV];
    float rbeta = 0.0f;
    auto load_raw = [&](int64_t ch) {
        const int64_t t0 = ch * kChunk;
        const int L = (int)((T_ - t0) < kChunk ? (T_ - t0) : kChunk);
        const int64_t tok0 = ((int64_t)b * T_ + t0) * H + h;
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            const int tl = tg * TPT + i;
            const int tc = tl < L ? tl : L - 1;          // clamp: never read past the end
            const int64_t e = (tok0 + (int64_t)tc * H) * DK + 4 * cq;
            rg[i] = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(gp + e));
            rk[i] = *reinterpret_cast<const T4 *>(kp + e);
            rq[i] = *reinterpret_cast<const T4 *>(qp + e);
        }
#pragma unroll
        for (int i = 0; i < TPV; ++i) {
            const int tl = tv * TPV + i;
            const int tc = tl < L ? tl : L - 1;
            rv[i] = *reinterpret_cast<const T4 *>(vp + (tok0 + (int64_t)tc * H) * DV + vcol0 + 4 * vq);
        }
        if (tid < 64) rbeta = to_f32(bp[tok0 + (int64_t)(tid < L ? tid : L - 1) * H]);
    };

    // ---- state: fp32 accumulator tiles of the owned column blocks ----------
    floatx4 sacc[NOWN][NCB];
#pragma unroll
    for (int m = 0; m < NOWN; ++m) {
        const int nb = wave + 4 * m;
        if (nb < NSB) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = 16 * cb + lg4 + j, n = vcol0 + 16 * nb + lr;
                    sacc[m][cb][j] = a.S0 ? a.S0[((int64_t)bh * DK + c) * DV + n] : 0.0f;
                }
                store4v(sST + (16 * nb + lr) * LDK + 16 * cb + lg4, sacc[m][cb]);
            }
        }
    }

    load_raw(0);
    for (int64_t ch = 0; ch < nchunk; ++ch) {
        const int64_t t0 = ch * kChunk;
        const int L = (int)((T_ - t0) < kChunk ? (T_ - t0) : kChunk);
        const int64_t tok0 = ((int64_t)b * T_ + t0) * H + h;
        const int I = wave;                              // this wave's subtile

        // ---- A1: running log-decay inside the subtile (in-wave scan) --------
        floatx4 lam[TPT];
        floatx4 run = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            const bool ok = tg * TPT + i < L;
            run += ok ? rg[i] : floatx4{0, 0, 0, 0};
            lam[i] = run;
        }
        floatx4 pre = {0, 0, 0, 0};
#pragma unroll
        for (int s = 1; s < 64 / NQ; ++s) {
            floatx4 other;
#pragma unroll
            for (int j = 0; j < 4; ++j) other[j] = __shfl(run[j], lane - s * NQ);
            if (pos >= s) pre += other;
        }
#pragma unroll
        for (int i = 0; i < TPT; ++i) lam[i] += pre;
        if (pos == 64 / NQ - 1)
            *reinterpret_cast<floatx4 *>(sLam + I * DK + 4 * cq) = lam[TPT - 1];
        if (tid < 64) sBeta[tid] = tid < L ? rbeta : 0.0f;
        __syncthreads();

        // ---- A2: decayed operand tiles -------------------------------------
        {
            const floatx4 L0 = *reinterpret_cast<const floatx4 *>(sLam + 4 * cq);
            const floatx4 L1 = *reinterpret_cast<const floatx4 *>(sLam + DK + 4 * cq);
            const floatx4 L2 = *reinterpret_cast<const floatx4 *>(sLam + 2 * DK + 4 * cq);
            const floatx4 L3 = *reinterpret_cast<const floatx4 *>(sLam + 3 * DK + 4 * cq);
            const floatx4 pre1 = L0, pre2 = L0 + L1, pre3 = pre2 + L2, pre4 = pre3 + L3;
            const floatx4 preI = I == 0 ? floatx4{0, 0, 0, 0} : I == 1 ? pre1 : I == 2 ? pre2 : pre3;
            const floatx4 LamI = I == 0 ? L0 : I == 1 ? L1 : I == 2 ? L2 : L3;
            const floatx4 preI1 = preI + LamI;             // b at the end of subtile I
            floatx4 ePre, eNegLam, eHat, eOff1, eOff2, eOff3;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                ePre[j] = __expf(preI[j]);                 // e^{b before subtile I}  <= 1
                eNegLam[j] = __expf(-LamI[j]);             // <= e^80
                eHat[j] = __expf(pre4[j] - preI1[j]);      // e^{b_C - b_end(I)}    <= 1
                // e^{sum_{I<K<I2} Lam_K}, used only for I2 > I
                eOff1[j] = __expf(I < 1 ? pre1[j] - preI1[j] : 0.0f);
                eOff2[j] = __expf(I < 2 ? pre2[j] - preI1[j] : 0.0f);
                eOff3[j] = __expf(I < 3 ? pre3[j] - preI1[j] : 0.0f);
            }
            if (I == 0 && pos == 0) {
                floatx4 ebc;
#pragma unroll
                for (int j = 0; j < 4; ++j) ebc[j] = __expf(pre4[j]);
                *reinterpret_cast<floatx4 *>(sEbC + 4 * cq) = ebc;
            }
            float ktb[4][TPT], kh[4][TPT];
#pragma unroll
            for (int i = 0; i < TPT; ++i) {
                const int tl = tg * TPT + i;               // token inside the chunk
                const int r = tl - 16 * I;                 // row inside the subtile
                const bool ok = tl < L;
                const floatx4 kv = ok ? to_f4(rk[i]) : floatx4{0, 0, 0, 0};
                const floatx4 qv = ok ? to_f4(rq[i]) : floatx4{0, 0, 0, 0};
                const float bt = sBeta[tl];
                floatx4 R, Et;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    R[j] = __expf(lam[i][j]);              // e^{lam_r}          in [e^-80, 1]
                    Et[j] = __expf(LamI[j] - lam[i][j]);   // e^{Lam_I - lam_r}  in [e^-75, 1]
                }
                const floatx4 kEt = kv * Et;
                store4v(sKr + tl * LDK + 4 * cq, kv * R * bt);
                store4v(sQr + tl * LDK + 4 * cq, qv * R);
                // column operands: diagonal pair (I,I) and off-diagonal pairs (I2,I), I2 > I
                store4v(sKc + (((I * (I + 1)) / 2 + I) * 16 + r) * LDK + 4 * cq, kEt * eNegLam);
                if (I < 1) store4v(sKc + ((1 + I) * 16 + r) * LDK + 4 * cq, kEt * eOff1);
                if (I < 2) store4v(sKc + ((3 + I) * 16 + r) * LDK + 4 * cq, kEt * eOff2);
                if (I < 3) store4v(sKc + ((6 + I) * 16 + r) * LDK + 4 * cq, kEt * eOff3);
                const floatx4 eb = R * ePre;               // e^{b_r} <= 1
                store4v(sQt + tl * LDK + 4 * cq, qv * eb);
                const floatx4 kt = kv * eb * bt, khv = kEt * eHat;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    ktb[j][i] = kt[j];
                    kh[j][i] = khv[j];
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                storeN<TPT>(sKtT + (4 * cq + j) * LDT + tg * TPT, ktb[j]);
                storeN<TPT>(sKhT + (4 * cq + j) * LDT + tg * TPT, kh[j]);
            }
            float vt[4][TPV];
#pragma unroll
            for (int i = 0; i < TPV; ++i) {
                const int tl = tv * TPV + i;
                const float bt = sBeta[tl];                // 0 past the end of the sequence
                const floatx4 vv = to_f4(rv[i]) * bt;
#pragma unroll
                for (int j = 0; j < 4; ++j) vt[j][i] = tl < L ? vv[j] : 0.0f;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) storeN<TPV>(sVT + (4 * vq + j) * LDT + tv * TPV, vt[j]);
        }
        if (ch + 1 < nchunk) load_raw(ch + 1);            // lands during stages B-E
        __syncthreads();

        // ---- B: A and P tiles (10 causal subtile pairs each) -----------------
        floatx4 sc[5];
        {
            const T *xs[5], *ys[5];
#pragma unroll
            for (int u = 0; u < 5; ++u) {
                const int ti = wave + 4 * u, p = ti >> 1;
                const int Ib = p >= 6 ? 3 : p >= 3 ? 2 : p >= 1 ? 1 : 0;
                sc[u] = floatx4{0, 0, 0, 0};
                xs[u] = sKc + p * 16 * LDK + lr * LDK + (lane >> 4) * (Mma<T>::kStep / 4);
                ys[u] = ((ti & 1) ? sQr : sKr) + (16 * Ib + lr) * LDK + (lane >> 4) * (Mma<T>::kStep / 4);
            }
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += Mma<T>::kStep)
#pragma unroll
                for (int u = 0; u < 5; ++u) Mma<T>::step(sc[u], xs[u] + k0, ys[u] + k0);
        }
        __syncthreads();   // region 1 is rewritten below
#pragma unroll
        for (int u = 0; u < 5; ++u) {
            const int ti = wave + 4 * u, p = ti >> 1;
            const int Ib = p >= 6 ? 3 : p >= 3 ? 2 : p >= 1 ? 1 : 0;
            const int J = p - (Ib * (Ib + 1)) / 2;
            const bool isP = ti & 1;
            floatx4 val;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int s = lg4 + j;                     // column inside block J
                const bool keep = (J < Ib) || (isP ? (s <= lr) : (s < lr));
                val[j] = keep ? sc[u][j] : 0.0f;
            }
            const int r = 16 * Ib + lr;
            if (isP) {
                store4v(sPh + r * LDT + 16 * J + lg4, val);
                if constexpr (kSplit) {
                    floatx4 lo;
#pragma unroll
                    for (int j = 0; j < 4; ++j) lo[j] = val[j] - (float)(bf16)val[j];
                    store4v(sPl + r * LDT + 16 * J + lg4, lo);
                }
            } else {
                store4v(sA + r * LDT + 16 * J + lg4, val);
            }
        }
        // zero the blocks above the diagonal of P (hi, lo) and X (read by the
        // rounded-up causal products)
        for (int e = tid; e < 6 * 64; e += 256) {
            const int blk = e >> 6, q4 = e & 63, rr = q4 >> 2, cc = (q4 & 3) * 4;
            const int Iu = blk < 3 ? 0 : blk < 5 ? 1 : 2;
            const int Ju = blk < 3 ? blk + 1 : blk < 5 ? blk - 1 : 3;
            const int off = (16 * Iu + rr) * LDT + 16 * Ju + cc;
            store4(sPh + off, 0.f, 0.f, 0.f, 0.f);
            if constexpr (kSplit) store4(sPl + off, 0.f, 0.f, 0.f, 0.f);
            store4(sXr + off, 0.f, 0.f, 0.f, 0.f);
        }
        __syncthreads();

        // ---- C: X = (I + A)^-1 ----------------------------------------------
        floatx4 xT;                                        // L(X_II^T) of this wave's block
        {
            const T tz = T(0);
            auto addI = [&](floatx4 m) {
#pragma unroll
                for (int j = 0; j < 4; ++j) m[j] += (lg4 + j == lr) ? 1.0f : 0.0f;
                return m;
            };
            const floatx4 z4 = {0, 0, 0, 0};
            // N = -A_II in both layouts
            const floatx4 nT = -lds_load4(sA + (16 * I + lr) * LDT + 16 * I + lg4);
            floatx4 n;
#pragma unroll
            for (int j = 0; j < 4; ++j) n[j] = -to_f32(sA[(16 * I + lg4 + j) * LDT + 16 * I + lr]);
            const floatx4 n2 = mma16(tz, nT, n, z4);
            const floatx4 n2T = mma16(tz, n, nT, z4);
            const floatx4 n4 = mma16(tz, n2T, n2, z4);
            const floatx4 n4T = mma16(tz, n2, n2T, z4);
            const floatx4 n8 = mma16(tz, n4T, n4, z4);
            const floatx4 p1 = mma16(tz, addI(nT), addI(n2), z4);
            const floatx4 p1T = mma16(tz, addI(n2), addI(nT), z4);
            (void)p1;
            const floatx4 p2T = mma16(tz, addI(n4), p1T, z4);
            const floatx4 p2 = mma16(tz, p1T, addI(n4), z4);
            (void)p2;
            const floatx4 x = mma16(tz, p2T, addI(n8), z4);
            xT = mma16(tz, addI(n8), p2T, z4);
            store4v(sXc + (16 * I + lr) * LDT + 16 * I + lg4, x);
            store4v(sXr + (16 * I + lr) * LDT + 16 * I + lg4, xT);
            __syncthreads();
            // blocks below the diagonal, one level per barrier:
            // X_IJ = -X_II sum_{K=J}^{I-1} A_IK X_KJ, computed by the wave of row block I
#pragma unroll
            for (int d = 1; d < 4; ++d) {
                if (I >= d) {
                    const int J = I - d;
                    floatx4 y = z4;
                    for (int K = J; K < I; ++K)
                        y = mma16(tz, lds_load4(sA + (16 * I + lr) * LDT + 16 * K + lg4),
                                  lds_load4(sXc + (16 * J + lr) * LDT + 16 * K + lg4), y);
                    const floatx4 xij = -mma16(tz, xT, y, z4);
                    const floatx4 xijT = -mma16(tz, y, xT, z4);
                    store4v(sXc + (16 * J + lr) * LDT + 16 * I + lg4, xij);
                    store4v(sXr + (16 * I + lr) * LDT + 16 * J + lg4, xijT);
                }
                __syncthreads();
            }
        }

        // ---- D: -W = -X (beta K~) into LDS; U' = X (beta V) into registers ----
        {
            floatx4 wacc[NCB];
            const T *xs = sXr + (16 * I + lr) * LDT + (lane >> 4) * (Mma<T>::kStep / 4);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) wacc[cb] = floatx4{0, 0, 0, 0};
            const int KI = kround<T>(I);
            for (int k0 = 0; k0 < KI; k0 += Mma<T>::kStep)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    Mma<T>::step(wacc[cb],
                                 sKtT + (16 * cb + lr) * LDT + (lane >> 4) * (Mma<T>::kStep / 4) + k0,
                                 xs + k0);
            // lane holds W^T[c = 16cb + lg4 + j][r = 16I + lr]
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                store4v(sWn + (16 * I + lr) * LDK + 16 * cb + lg4, -wacc[cb]);
        }
        floatx4 uacc[NOWN][4];
#pragma unroll
        for (int m = 0; m < NOWN; ++m) {
            const int nb = wave + 4 * m;
            if (nb < NSB) {
#pragma unroll
                for (int Is = 0; Is < 4; ++Is) {
                    uacc[m][Is] = floatx4{0, 0, 0, 0};
                    tile_mma<T>(uacc[m][Is], sXr + 16 * Is * LDT, LDT, sVT + 16 * nb * LDT, LDT,
                                kround<T>(Is), lane);
                }
            }
        }
        __syncthreads();

        // ---- E: state pass of the owned column blocks (no barrier) ----------
#pragma unroll
        for (int m = 0; m < NOWN; ++m) {
            const int nb = wave + 4 * m;
            if (nb >= NSB) continue;
            // U = U' - W S, kept as hi + lo (tokens contiguous)
#pragma unroll
            for (int Is = 0; Is < 4; ++Is) {
                tile_mma<T>(uacc[m][Is], sWn + 16 * Is * LDK, LDK, sST + 16 * nb * LDK, LDK, DK,
                            lane);
                store4v(sUh + (16 * nb + lr) * LDT + 16 * Is + lg4, uacc[m][Is]);
                if constexpr (kSplit) {
                    floatx4 lo;
#pragma unroll
                    for (int j = 0; j < 4; ++j) lo[j] = uacc[m][Is][j] - (float)(bf16)uacc[m][Is][j];
                    store4v(sUl + (16 * nb + lr) * LDT + 16 * Is + lg4, lo);
                }
            }
            wave_lds_sync();
            // O = Q~ S + P U for the 64 rows of this column block
#pragma unroll
            for (int Ir = 0; Ir < 4; ++Ir) {
                floatx4 acc = {0, 0, 0, 0};
                tile_mma<T>(acc, sST + 16 * nb * LDK, LDK, sQt + 16 * Ir * LDK, LDK, DK, lane);
                const int KI = kround<T>(Ir);
                tile_mma<T>(acc, sUh + 16 * nb * LDT, LDT, sPh + 16 * Ir * LDT, LDT, KI, lane);
                if constexpr (kSplit) {
                    tile_mma<T>(acc, sUl + 16 * nb * LDT, LDT, sPh + 16 * Ir * LDT, LDT, KI, lane);
                    tile_mma<T>(acc, sUh + 16 * nb * LDT, LDT, sPl + 16 * Ir * LDT, LDT, KI, lane);
                }
                const int r = 16 * Ir + lr;
                if (r < L)
                    store4v(op + (tok0 + (int64_t)r * H) * DV + vcol0 + 16 * nb + lg4, acc);
            }
            // S <- Diag(e^{b_C}) S + K^^T U
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const floatx4 e = *reinterpret_cast<const floatx4 *>(sEbC + 16 * cb + lg4);
                sacc[m][cb] *= e;
                tile_mma<T>(sacc[m][cb], sKhT + 16 * cb * LDT, LDT, sUh + 16 * nb * LDT, LDT,
                            kChunk, lane);
            }
            wave_lds_sync();   // this wave's reads of the old state copy are done
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                store4v(sST + (16 * nb + lr) * LDK + 16 * cb + lg4, sacc[m][cb]);
        }
    }

    if (a.ST) {
#pragma unroll
        for (int m = 0; m < NOWN; ++m) {
            const int nb = wave + 4 * m;
            if (nb >= NSB) continue;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = 16 * cb + lg4 + j, n = vcol0 + 16 * nb + lr;
                    a.ST[((int64_t)bh * DK + c) * DV + n] = sacc[m][cb][j];
                }
        }
    }
}

// dv-slice width per workgroup: four 16-column blocks (one per wave) where
// the LDS plan allows it.
static int slice_width(int dk, int dv, int is_bf16) {
    int nv = 64;
    if (!is_bf16 && dk == 64) nv = 32;   // fp32 tiles at dk = 64 leave room for 32 columns
    if (nv > dv) nv = dv;
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
    case 32064: return launch_inst<float, 32, 64>(args, nblocks, s);
    case 64032: return launch_inst<float, 64, 32>(args, nblocks, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
