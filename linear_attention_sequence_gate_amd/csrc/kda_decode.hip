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
// ~115 kflop), so the design goal is a single coalesced sweep of the state:
//  - a workgroup of TPB threads (512 at d = 128) holds one head's state in
//    registers, each thread a float4 column group over DK / (TPB / (DV/4))
//    rows, between the reduction and the write;
//  - the grid is persistent (about four workgroups per CU): a workgroup walks
//    heads blockIdx.x, blockIdx.x + gridDim.x, ... and issues the loads of its
//    next head's state before writing the current one, so reads of one head
//    overlap the writes of the previous;
//  - state reads and writes bypass the caches (nontemporal): every byte is
//    touched exactly once per step.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

template <typename T>
__device__ __forceinline__ float ld1(const T *p) { return to_f32(*p); }

__device__ __forceinline__ floatx4 ld_state(const floatx4 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_state(floatx4 *p, floatx4 v) { __builtin_nontemporal_store(v, p); }

template <int DK, int DV> struct DecodeShape {
    static constexpr int TPB = DK * DV / 4 < 512 ? DK * DV / 4 : 512;   // threads per head
    static constexpr int NCG = DV / 4;          // float4 column groups
    static constexpr int RG = TPB / NCG;        // row groups
    static constexpr int ROWS = DK / RG;        // rows per thread
    static constexpr int NWV = TPB / 64;        // waves
    static_assert(ROWS >= 1 && DK % RG == 0 && TPB % 64 == 0 && NCG <= 64, "decode shape");
};

template <typename T, int DK, int DV, bool POOLED>
__global__ __launch_bounds__((DecodeShape<DK, DV>::TPB)) void decode_step_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ z, const float *__restrict__ A, const T *__restrict__ beta,
    float *__restrict__ state, T *__restrict__ o, int H, int64_t NH,
    const int *__restrict__ slots, int64_t n_slots) {
    using Sh = DecodeShape<DK, DV>;
    constexpr int NCG = Sh::NCG, RG = Sh::RG, ROWS = Sh::ROWS, NWV = Sh::NWV;

    __shared__ float sAlpha[DK], sK[DK], sQ[DK];
    __shared__ float sV[DV];
    __shared__ floatx4 sRed[NWV][2][NCG];
    __shared__ float sKq[NWV];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = tid % NCG, rg = tid / NCG;
    int64_t nh = blockIdx.x;                     // the grid never exceeds NH
    // the state of head nh: row nh of the state array, or with a slot table
    // row slots[n] * H + h of the pool; -1 for a slot outside the pool (the
    // head is skipped: nothing of it is read or written but q..beta)
    auto state_row = [&](int64_t i) -> int64_t {
        if constexpr (!POOLED) return i;
        const int64_t n = i / H;
        const int sl = slots[n];
        return (sl >= 0 && sl < n_slots) ? (int64_t)sl * H + (i - n * H) : -1;
    };

    // this head's state and small inputs are in registers when an iteration
    // starts; the next head's are requested before this head's write
    floatx4 s[ROWS], sn[ROWS];
    float kk = 0.0f, qq = 0.0f, zz = 0.0f, vv = 0.0f, bt;
    auto load_small = [&](int64_t n, float &k_, float &q_, float &z_, float &v_, float &b_) {
        if (tid < DK) {
            const int64_t off = n * DK + tid;
            k_ = ld1(k + off);
            q_ = ld1(q + off);
            z_ = ld1(z + off);
        }
        if (tid < DV) v_ = ld1(v + n * DV + tid);
        b_ = ld1(beta + n);
    };
    int64_t row = state_row(nh);
    {
        // a skipped head's address is kept inside the pool (row 0) as well
        const floatx4 *Sp = reinterpret_cast<const floatx4 *>(state + (row >= 0 ? row : 0) * (int64_t)(DK * DV));
#pragma unroll
        for (int i = 0; i < ROWS; ++i)
            s[i] = row >= 0 ? ld_state(Sp + (rg + RG * i) * NCG + cg) : floatx4{0, 0, 0, 0};
        load_small(nh, kk, qq, zz, vv, bt);
    }
    for (; nh < NH; nh += gridDim.x) {
        const int h = (int)(nh % H);
        const bool live = row >= 0;
        floatx4 *Sp = reinterpret_cast<floatx4 *>(state + (live ? row : 0) * (int64_t)(DK * DV));

        // per-channel gate, key and query, and the partial k . q
        float kq = 0.0f;
        if (tid < DK) {
            sAlpha[tid] = expf(gate_value(A[h * DK + tid], zz));
            sK[tid] = kk;
            sQ[tid] = qq;
            kq = kk * qq;
        }
        if (tid < DV) sV[tid] = vv;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) kq += __shfl_xor(kq, m);
        if (lane == 0) sKq[wave] = kq;
        __syncthreads();

        // decay the rows and accumulate the two projections
        floatx4 r1 = {0, 0, 0, 0}, r2 = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < ROWS; ++i) {
            const int c = rg + RG * i;
            s[i] *= sAlpha[c];
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
        // ... then across the waves
        if (lane < NCG) {
            sRed[wave][0][cg] = r1;
            sRed[wave][1][cg] = r2;
        }
        __syncthreads();
        r1 = sRed[0][0][cg];
        r2 = sRed[0][1][cg];
        float kappa = sKq[0];
#pragma unroll
        for (int w = 1; w < NWV; ++w) {
            r1 += sRed[w][0][cg];
            r2 += sRed[w][1][cg];
            kappa += sKq[w];
        }
        floatx4 u;
#pragma unroll
        for (int j = 0; j < 4; ++j) u[j] = bt * (sV[4 * cg + j] - r1[j]);

        // next head's state in flight before this head's write
        const int64_t nxt = nh + gridDim.x;
        const int64_t nrow = nxt < NH ? state_row(nxt) : -1;
        float nk = 0.0f, nq = 0.0f, nz = 0.0f, nv = 0.0f, nb = 0.0f;
        if (nxt < NH) {
            const floatx4 *Np = reinterpret_cast<const floatx4 *>(state + (nrow >= 0 ? nrow : 0) * (int64_t)(DK * DV));
#pragma unroll
            for (int i = 0; i < ROWS; ++i)
                sn[i] = nrow >= 0 ? ld_state(Np + (rg + RG * i) * NCG + cg) : floatx4{0, 0, 0, 0};
            load_small(nxt, nk, nq, nz, nv, nb);
        }
        // the new state, in place, and the output
        if (live) {
#pragma unroll
            for (int i = 0; i < ROWS; ++i) {
                const int c = rg + RG * i;
                st_state(Sp + c * NCG + cg, s[i] + sK[c] * u);
            }
            if (rg == 0) {
                const floatx4 ov = r2 + kappa * u;
                store4(o + nh * DV + 4 * cg, ov[0], ov[1], ov[2], ov[3]);
            }
        }
        __syncthreads();                         // the LDS tables are rewritten next
#pragma unroll
        for (int i = 0; i < ROWS; ++i) s[i] = sn[i];
        kk = nk; qq = nq; zz = nz; vv = nv; bt = nb;
        row = nrow;
    }
}

template <typename T, int DK>
static hipError_t decode_dv(const void *q, const void *k, const void *v, const void *z,
                            const float *A, const void *beta, float *state, void *o,
                            int64_t NH, int H, int dv, const int *slots, int64_t n_slots,
                            hipStream_t s) {
    // persistent grid: about four workgroups per CU, never more than NH
    const unsigned grid = (unsigned)(NH < 1024 ? NH : 1024);
#define KDA_DECODE(DV)                                                                      \
    if (slots)                                                                               \
        hipLaunchKernelGGL((decode_step_kernel<T, DK, DV, true>), dim3(grid),                \
                           dim3(DecodeShape<DK, DV>::TPB), 0, s, (const T *)q, (const T *)k, \
                           (const T *)v, (const T *)z, A, (const T *)beta, state, (T *)o, H, \
                           NH, slots, n_slots);                                              \
    else                                                                                     \
        hipLaunchKernelGGL((decode_step_kernel<T, DK, DV, false>), dim3(grid),               \
                           dim3(DecodeShape<DK, DV>::TPB), 0, s, (const T *)q, (const T *)k, \
                           (const T *)v, (const T *)z, A, (const T *)beta, state, (T *)o, H, \
                           NH, nullptr, 0)
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
                            int64_t NH, int H, int dk, int dv, const int *slots, int64_t n_slots,
                            hipStream_t s) {
    switch (dk) {
    case 32: return decode_dv<T, 32>(q, k, v, z, A, beta, state, o, NH, H, dv, slots, n_slots, s);
    case 64: return decode_dv<T, 64>(q, k, v, z, A, beta, state, o, NH, H, dv, slots, n_slots, s);
    case 128: return decode_dv<T, 128>(q, k, v, z, A, beta, state, o, NH, H, dv, slots, n_slots, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_step(const void *q, const void *k, const void *v, const void *z,
                              const float *A, const void *beta, float *state, void *o,
                              int64_t N, int64_t H, int dk, int dv, int is_bf16, const int *slots,
                              int64_t n_slots, hipStream_t s) {
    const int64_t NH = N * H;
    if (is_bf16)
        return decode_dk<bf16>(q, k, v, z, A, beta, state, o, NH, (int)H, dk, dv, slots, n_slots, s);
    return decode_dk<float>(q, k, v, z, A, beta, state, o, NH, (int)H, dk, dv, slots, n_slots, s);
}

// Zero the states of the listed slots of a pool [n_slots, H, dk, dv] (slots
// outside the pool are skipped).  One thread per 4 floats.
__global__ __launch_bounds__(256) void pool_reset_kernel(float *__restrict__ pool,
                                                         const int *__restrict__ slots, int64_t n,
                                                         int64_t n_slots, int64_t per_slot4) {
    const int64_t total = n * per_slot4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t r = i / per_slot4, e = i - r * per_slot4;
        const int sl = slots[r];
        if (sl < 0 || sl >= n_slots) continue;
        reinterpret_cast<floatx4 *>(pool)[(int64_t)sl * per_slot4 + e] = floatx4{0, 0, 0, 0};
    }
}

hipError_t launch_pool_reset(float *pool, const int *slots, int64_t n, int64_t n_slots,
                             int64_t per_slot, hipStream_t s) {
    const int64_t per4 = per_slot / 4, total = n * per4;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(pool_reset_kernel, dim3((unsigned)blocks), dim3(256), 0, s, pool, slots, n,
                       n_slots, per4);
    return hipGetLastError();
}

}  // namespace kda
