// C ABI of libkda: argument validation, error reporting, dispatch to the
// kernel launchers.  Declarations and the contract live in include/kda.h.
#include "kda.h"

#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "kda_launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return KDA_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dim(int64_t d) { return d == 32 || d == 64 || d == 128; }

// a * b * ... without signed overflow, capped well below INT64_MAX
bool mul_ok(int64_t &acc, int64_t x) {
    int64_t r;
    if (__builtin_mul_overflow(acc, x, &r) || r > (int64_t(1) << 60)) return false;
    acc = r;
    return true;
}

int check_dtype(int dtype) {
    if (dtype != KDA_F32 && dtype != KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "unknown dtype %d (expected KDA_F32=0 or KDA_BF16=1)", dtype);
    return KDA_OK;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// pool [n_slots, H, dk, dv] and slot table checks shared by the pooled entry points
int check_pool(const char *who, const float *pool, const int32_t *slots, int64_t n_slots,
               int64_t H, int64_t dk, int64_t dv) {
    if (!pool || !slots) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: null state_pool or slots", who);
    if (n_slots <= 0 || H <= 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: sizes must be positive", who);
    if (!valid_dim(dk) || !valid_dim(dv))
        return fail(KDA_ERR_UNSUPPORTED, "%s: dk=%lld dv=%lld must be in {32,64,128}", who,
                    (long long)dk, (long long)dv);
    int64_t np = n_slots;
    if (!mul_ok(np, H) || !mul_ok(np, dk) || !mul_ok(np, dv))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: pool size overflows", who);
    if (n_slots * H > 0x7fffffffLL)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: n_slots*H too large", who);
    if (!aligned16(pool)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: state_pool must be 16-byte aligned", who);
    if (reinterpret_cast<uintptr_t>(slots) & 3u)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: slots must be 4-byte aligned", who);
    return KDA_OK;
}

}  // namespace

extern "C" {

const char *kda_last_error(void) { return g_last_error.c_str(); }

const char *kda_version(void) { return "libkda 0.1 (gfx950)"; }

int kda_gate(const void *z, const float *A, float *g, int64_t B, int64_t T, int64_t H, int64_t dk,
             int dtype, void *stream) {
    if (int e = check_dtype(dtype)) return e;
    if (!z || !A || !g) return fail(KDA_ERR_INVALID_ARGUMENT, "kda_gate: null pointer");
    if (B <= 0 || T <= 0 || H <= 0 || dk <= 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_gate: sizes must be positive");
    if (!valid_dim(dk)) return fail(KDA_ERR_UNSUPPORTED, "kda_gate: dk=%lld not in {32,64,128}", (long long)dk);
    int64_t n = B;
    if (!mul_ok(n, T) || !mul_ok(n, H) || !mul_ok(n, dk))
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_gate: element count overflows");
    if (H * dk > (int64_t(1) << 28))
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_gate: H*dk=%lld too large", (long long)(H * dk));
    if (!aligned16(z) || !aligned16(A) || !aligned16(g))
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_gate: pointers must be 16-byte aligned");
    if (static_cast<const void *>(g) == z)
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_gate: g must not alias z");
    hipError_t e = kda::launch_gate(z, A, g, n, (int)H, (int)dk, dtype == KDA_BF16,
                                    static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "kda_gate launch");
    return ok();
}

size_t kda_gate_bwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t dk) {
    if (B <= 0 || T <= 0 || H <= 0 || !valid_dim(dk)) return 0;
    int64_t n = B;
    if (!mul_ok(n, T) || !mul_ok(n, H) || !mul_ok(n, dk) || H * dk > (int64_t(1) << 28)) return 0;
    return kda::gate_bwd_workspace_bytes(B * T, (int)(H * dk));
}

int kda_gate_bwd(const void *z, const float *A, const float *dg, float *dz, float *dA,
                 void *workspace, size_t workspace_bytes, int64_t B, int64_t T, int64_t H,
                 int64_t dk, int dtype, void *stream) {
    const char *who = "kda_gate_bwd";
    if (int e = check_dtype(dtype)) return e;
    if (!z || !A || !dg || !dz || !dA || !workspace)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: null pointer", who);
    if (B <= 0 || T <= 0 || H <= 0 || dk <= 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: sizes must be positive", who);
    if (!valid_dim(dk)) return fail(KDA_ERR_UNSUPPORTED, "%s: dk=%lld not in {32,64,128}", who, (long long)dk);
    int64_t n = B;
    if (!mul_ok(n, T) || !mul_ok(n, H) || !mul_ok(n, dk))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: element count overflows", who);
    if (H * dk > (int64_t(1) << 28))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: H*dk=%lld too large", who, (long long)(H * dk));
    const size_t need = kda_gate_bwd_workspace_size(B, T, H, dk);
    if (workspace_bytes < need)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: needs a workspace of %zu bytes", who, need);
    const void *ptrs[] = {z, A, dg, dz, dA, workspace};
    for (const void *p : ptrs)
        if (!aligned16(p)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: pointers must be 16-byte aligned", who);
    const void *outs[] = {dz, dA, workspace};
    const void *ins[] = {z, A, dg};
    for (const void *po : outs)
        for (const void *pi : ins)
            if (po == pi) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: outputs must not alias inputs", who);
    if (static_cast<const void *>(dz) == dA || static_cast<const void *>(dz) == workspace ||
        static_cast<const void *>(dA) == workspace)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: outputs must not alias each other", who);
    hipError_t e = kda::launch_gate_bwd(z, A, dg, dz, dA, static_cast<float *>(workspace), B * T,
                                        (int)H, (int)dk, dtype == KDA_BF16,
                                        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "kda_gate_bwd launch");
    return ok();
}

// The workspace: the range-check counter (256 bytes), then the buffers of the
// sequence split when it is used.
static constexpr size_t kCounterBytes = 256;

// The workgroup layout the flags ask for: 1 one per chain, 0 one per
// 64-column slice (also the position-pair path's), -1 the library's choice.
static int layout_request(unsigned flags) {
    if (flags & KDA_FLAG_WORKGROUP_PER_CHAIN) return 1;
    if ((flags & KDA_FLAG_WORKGROUP_PER_SLICE) || (flags & KDA_FLAG_PAIRWISE_DIAGONAL)) return 0;
    return -1;
}

size_t kda_chunk_fwd_workspace_size_segments(int64_t B, int64_t T, int64_t H, int64_t dk,
                                             int64_t dv, int dtype, int nseg) {
    if (B <= 0 || T <= 0 || H <= 0 || !valid_dim(dk) || !valid_dim(dv)) return 0;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return 0;
    if (nseg < 0 || nseg > 255) return 0;
    const bool bf = dtype == KDA_BF16;
    // fp32 inputs at dk = 128: the fp32 16-token path's per-chunk buffers
    if (!kda::chunk_fwd_supported((int)dk, (int)dv, bf))
        return kCounterBytes + kda::cb_prefill_workspace_bytes(B, T, H, (int)dk);
    if (!kda::seq_split_supported((int)dk, (int)dv, bf)) return kCounterBytes;
    if (nseg != 0) return kCounterBytes + (nseg >= 2 ? kda::seq_split_workspace(B, T, H, (int)dk, (int)dv, nseg) : 0);
    // the library's count, for either scheme (with and without
    // KDA_FLAG_SPLIT_FULL_RERUN) and any workgroup layout flag: the same
    // buffers, sized for the largest
    size_t ws = 0;
    for (int rerun = 0; rerun < 2; ++rerun)
        for (int layout = -1; layout <= 1; ++layout) {
            const int P = kda::seq_split_auto(B, T, H, (int)dk, (int)dv, bf, rerun, layout);
            const size_t w = P >= 2 ? kda::seq_split_workspace(B, T, H, (int)dk, (int)dv, P) : 0;
            if (w > ws) ws = w;
        }
    return kCounterBytes + ws;
}

int kda_chunk_fwd_auto_segments(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                int dtype) {
    if (B <= 0 || T <= 0 || H <= 0 || !valid_dim(dk) || !valid_dim(dv)) return 0;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return 0;
    const int P = kda::seq_split_auto(B, T, H, (int)dk, (int)dv, dtype == KDA_BF16, 0, -1);
    return P >= 2 ? kda::seq_split_effective(T, P) : 1;
}

size_t kda_chunk_fwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                    int dtype) {
    return kda_chunk_fwd_workspace_size_segments(B, T, H, dk, dv, dtype, 0);
}

int kda_chunk_fwd_plan(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int dtype,
                       unsigned flags, int *segments, int *per_chain, int *guarded) {
    const char *who = "kda_chunk_fwd_plan";
    if (int e = check_dtype(dtype)) return e;
    if (!segments || !per_chain || !guarded) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: null pointer", who);
    if (B <= 0 || T <= 0 || H <= 0 || dk <= 0 || dv <= 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: sizes must be positive", who);
    if (!valid_dim(dk) || !valid_dim(dv))
        return fail(KDA_ERR_UNSUPPORTED, "%s: dk=%lld dv=%lld must be in {32,64,128}", who,
                    (long long)dk, (long long)dv);
    if (flags & ~unsigned(KDA_FLAG_CHECK_RANGE | KDA_FLAG_PAIRWISE_DIAGONAL | KDA_FLAG_SEGMENTS_MASK |
                          KDA_FLAG_SPLIT_FULL_RERUN | KDA_FLAG_WORKGROUP_PER_CHAIN |
                          KDA_FLAG_WORKGROUP_PER_SLICE))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown flag bits 0x%x", who, flags);
    const bool bf = dtype == KDA_BF16;
    const bool pipe = kda::seq_split_supported((int)dk, (int)dv, bf);
    const int layout = layout_request(flags);
    const int req_seg = (int)((flags & KDA_FLAG_SEGMENTS_MASK) >> KDA_FLAG_SEGMENTS_SHIFT);
    if ((flags & KDA_FLAG_WORKGROUP_PER_CHAIN) && (flags & KDA_FLAG_WORKGROUP_PER_SLICE))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: the two workgroup layout flags exclude each other", who);
    if ((flags & KDA_FLAG_WORKGROUP_PER_CHAIN) &&
        (!kda::seq_wide_supported((int)dk, (int)dv, bf) || (flags & KDA_FLAG_PAIRWISE_DIAGONAL)))
        return fail(KDA_ERR_UNSUPPORTED, "%s: one workgroup per chain needs bf16 inputs, dk = dv = 128 "
                    "and no KDA_FLAG_PAIRWISE_DIAGONAL", who);
    if (((flags & KDA_FLAG_PAIRWISE_DIAGONAL) || req_seg >= 2) && !pipe)
        return fail(KDA_ERR_UNSUPPORTED, "%s: a sequence split or the position-pair path needs bf16 "
                    "inputs, dk = 128, dv in {64, 128}", who);
    const int rerun = (flags & KDA_FLAG_SPLIT_FULL_RERUN) ? 1 : 0;
    int nseg = req_seg == 0 ? kda::seq_split_auto(B, T, H, (int)dk, (int)dv, bf, rerun, layout) : req_seg;
    nseg = pipe && nseg >= 2 ? kda::seq_split_effective(T, nseg) : 1;
    *segments = nseg;
    *per_chain = kda::seq_layout(B, T, H, (int)dk, (int)dv, bf, rerun, nseg, layout);
    *guarded = 0;
    if (req_seg == 0 && !rerun && nseg == 2) {
        const int fb = kda::seq_layout(B, T, H, (int)dk, (int)dv, bf, 0, 1, layout);
        *guarded = kda::seq_split_guarded(B, T, H, (int)dk, (int)dv, bf, nseg, *per_chain, fb) ? 1 : 0;
    }
    return ok();
}

// kda_chunk_fwd_gated: shapes without the fused gate stage g at the start of
// the workspace, B*T*H*dk fp32 rounded up to 256 bytes
static size_t gate_stage_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int dtype) {
    if (kda::seq_split_supported((int)dk, (int)dv, dtype == KDA_BF16)) return 0;
    int64_t n = B;
    if (!mul_ok(n, T) || !mul_ok(n, H) || !mul_ok(n, dk) || !mul_ok(n, 4)) return SIZE_MAX;
    return ((size_t)n + 255) / 256 * 256;
}

size_t kda_chunk_fwd_gated_workspace_size(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                          int dtype) {
    const size_t base = kda_chunk_fwd_workspace_size(B, T, H, dk, dv, dtype);
    if (base == 0) return 0;
    const size_t gb = gate_stage_bytes(B, T, H, dk, dv, dtype);
    return gb == SIZE_MAX ? 0 : gb + base;
}

}  // extern "C"

namespace {

// Every chunked-prefill entry point: kda_chunk_fwd, kda_chunk_fwd_gated (z,
// Ag set: the gate is evaluated inside the call), and the pooled and
// variable-length forms (slots, cu_seqlens); `who` names the entry point in
// errors.  Validation ends before the first HIP call.
int chunk_fwd_impl(const char *who, const void *q, const void *k, const void *v, const float *g,
                   const void *beta, const float *initial_state, float *final_state, void *o,
                   void *workspace, size_t workspace_bytes, int64_t B, int64_t T, int64_t H,
                   int64_t dk, int64_t dv, int dtype, unsigned flags, const int32_t *slots,
                   int64_t n_slots, const int64_t *cu_seqlens, const void *z, const float *Ag,
                   void *stream) {
    if (int e = check_dtype(dtype)) return e;
    // gated: g comes from (z, A) inside the call
    const bool gated = z != nullptr || Ag != nullptr;
    if (!q || !k || !v || !beta || !o || (gated ? (!z || !Ag) : !g))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: null pointer (q, k, v, %s, beta, o are required)", who,
                    gated ? "z, A" : "g");
    if (B <= 0 || T <= 0 || H <= 0 || dk <= 0 || dv <= 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: sizes must be positive", who);
    if (!valid_dim(dk) || !valid_dim(dv))
        return fail(KDA_ERR_UNSUPPORTED, "%s: dk=%lld dv=%lld must be in {32,64,128}", who,
                    (long long)dk, (long long)dv);
    // fp32 inputs at dk = 128 run the fp32 16-token path (the reverse mode's
    // chunk preparation and forward pass with outputs), [B, T, H] layout only
    const bool cbpath = !kda::chunk_fwd_supported((int)dk, (int)dv, dtype == KDA_BF16);
    if (cbpath && cu_seqlens)
        return fail(KDA_ERR_UNSUPPORTED, "%s: fp32 inputs with dk = 128 take the [B, T, H] layout "
                    "(no packed sequences)", who);
    if (flags & ~unsigned(KDA_FLAG_CHECK_RANGE | KDA_FLAG_PAIRWISE_DIAGONAL | KDA_FLAG_SEGMENTS_MASK |
                          KDA_FLAG_SPLIT_FULL_RERUN | KDA_FLAG_WORKGROUP_PER_CHAIN |
                          KDA_FLAG_WORKGROUP_PER_SLICE))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown flag bits 0x%x", who, flags);
    if ((flags & KDA_FLAG_WORKGROUP_PER_CHAIN) && (flags & KDA_FLAG_WORKGROUP_PER_SLICE))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: KDA_FLAG_WORKGROUP_PER_CHAIN and "
                    "KDA_FLAG_WORKGROUP_PER_SLICE exclude each other", who);
    const bool is_bf16 = dtype == KDA_BF16;
    const bool pairwise = (flags & KDA_FLAG_PAIRWISE_DIAGONAL) != 0;
    if (pairwise && !kda::seq_split_supported((int)dk, (int)dv, is_bf16))
        return fail(KDA_ERR_UNSUPPORTED, "%s: the position-pair diagonal path needs bf16 inputs, dk = 128, "
                    "dv in {64, 128}", who);
    if ((flags & KDA_FLAG_WORKGROUP_PER_CHAIN) &&
        !(kda::seq_split_supported((int)dk, (int)dv, is_bf16) && dv == 128 && !pairwise))
        return fail(KDA_ERR_UNSUPPORTED, "%s: one workgroup per chain needs bf16 inputs, dk = dv = 128 "
                    "and no KDA_FLAG_PAIRWISE_DIAGONAL", who);
    if (pairwise && (flags & KDA_FLAG_CHECK_RANGE))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: the position-pair diagonal path has no decay range to check", who);
    const int req_seg = (int)((flags & KDA_FLAG_SEGMENTS_MASK) >> KDA_FLAG_SEGMENTS_SHIFT);
    if (req_seg >= 2 && !kda::seq_split_supported((int)dk, (int)dv, is_bf16))
        return fail(KDA_ERR_UNSUPPORTED, "%s: a sequence split needs bf16 inputs, dk = 128, dv in {64, 128}", who);
    int64_t nk = B, nv = B, ns = B;
    if (!mul_ok(nk, T) || !mul_ok(nk, H) || !mul_ok(nk, dk) || !mul_ok(nv, T) || !mul_ok(nv, H) ||
        !mul_ok(nv, dv) || !mul_ok(ns, H) || !mul_ok(ns, dk) || !mul_ok(ns, dv))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: element count overflows", who);
    if (B * H > (int64_t(1) << 24))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: B*H=%lld too large", who, (long long)(B * H));
    // the kernel addresses the tokens of one 64-token chunk with 32-bit byte offsets
    if (H * (dk > dv ? dk : dv) * 64 * 4 >= (int64_t(1) << 32))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: H=%lld too large", who, (long long)H);
    const void *ptrs[] = {q, k, v, g, beta, initial_state, final_state, o, workspace, z, Ag};
    for (const void *p : ptrs)
        if (p && !aligned16(p))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: pointers must be 16-byte aligned", who);
    const void *ins[] = {q, k, v, g, beta, initial_state, z, Ag};
    for (const void *p : ins)
        if (p && p == o) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: o must not alias an input", who);
    if (gated && (flags & KDA_FLAG_CHECK_RANGE))
        return fail(KDA_ERR_INVALID_ARGUMENT,
                    "%s: g comes from the gate inside the call and lies in [-5, 0] by construction; "
                    "KDA_FLAG_CHECK_RANGE checks a caller's g", who);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the fused gate runs in the pipelined kernel; other shapes stage g in
    // the workspace with the gate kernel first
    const bool fused = gated && kda::seq_split_supported((int)dk, (int)dv, dtype == KDA_BF16);
    if (gated && !fused) {
        const size_t gb = gate_stage_bytes(B, T, H, dk, dv, dtype);
        if (!workspace || workspace_bytes < gb)
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: needs a workspace of %zu bytes for g", who,
                        kda_chunk_fwd_gated_workspace_size(B, T, H, dk, dv, dtype));
        float *gs = static_cast<float *>(workspace);
        const void *tens[] = {q, k, v, z, Ag, beta, initial_state, final_state, o};
        for (const void *p : tens)
            if (p == static_cast<const void *>(gs))
                return fail(KDA_ERR_INVALID_ARGUMENT, "%s: the workspace must not alias a tensor", who);
        hipError_t e = kda::launch_gate(z, Ag, gs, B * T * H * dk, (int)H, (int)dk, dtype == KDA_BF16, s);
        if (e != hipSuccess) return hip_fail(e, "kda_chunk_fwd_gated gate launch");
        g = gs;
        workspace = static_cast<char *>(workspace) + gb;
        workspace_bytes -= gb;
    }

    if (flags & KDA_FLAG_CHECK_RANGE) {
        if (!workspace || workspace_bytes < kda_chunk_fwd_workspace_size(B, T, H, dk, dv, dtype))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: KDA_FLAG_CHECK_RANGE needs a workspace of %zu bytes", who,
                        kda_chunk_fwd_workspace_size(B, T, H, dk, dv, dtype));
        unsigned int *bad = static_cast<unsigned int *>(workspace);
        hipError_t e = hipMemsetAsync(bad, 0, sizeof(unsigned int), s);
        if (e != hipSuccess) return hip_fail(e, "kda_chunk_fwd range check memset");
        e = kda::launch_range_check(g, B, T, H, dk, bad, s);
        if (e != hipSuccess) return hip_fail(e, "kda_chunk_fwd range check launch");
        unsigned int nbad = 0;
        e = hipMemcpyAsync(&nbad, bad, sizeof nbad, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_fail(e, "kda_chunk_fwd range check readback");
        if (nbad)
            return fail(KDA_ERR_RANGE, "%s: %u gate values or 16-token tile sums outside [-5,0] / [-80,0]", who,
                        nbad);
    }
    if (cbpath) {
        const size_t need = kCounterBytes + kda::cb_prefill_workspace_bytes(B, T, H, (int)dk);
        if (!workspace || workspace_bytes < need)
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: fp32 inputs with dk = 128 need a workspace of %zu bytes",
                        who, need);
        hipError_t e = kda::launch_chunk_fwd_cb(q, k, v, g, beta, initial_state, final_state, o,
                                                static_cast<char *>(workspace) + kCounterBytes,
                                                workspace_bytes - kCounterBytes, B, T, H, (int)dk,
                                                (int)dv, is_bf16, slots, n_slots, s);
        if (e != hipSuccess) return hip_fail(e, "kda_chunk_fwd launch");
        return ok();
    }
    // sequence split: requested, or picked for these sizes among the counts
    // whose buffers the workspace holds (none: one pass)
    const int rerun = (flags & KDA_FLAG_SPLIT_FULL_RERUN) ? 1 : 0;
    // workgroup layout: forced by a flag (the position-pair path runs per
    // slice), else chosen with the segment count
    const int layout = layout_request(flags);
    int nseg = req_seg == 0 ? kda::seq_split_auto(B, T, H, (int)dk, (int)dv, is_bf16, rerun, layout)
                            : req_seg;
    void *split_ws = nullptr;
    if (nseg >= 2) {
        const size_t need = kda_chunk_fwd_workspace_size_segments(B, T, H, dk, dv, dtype, nseg);
        if (workspace && workspace_bytes >= need) {
            split_ws = static_cast<char *>(workspace) + kCounterBytes;
        } else if (req_seg >= 2) {
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: a %d-segment split needs a workspace of %zu bytes", who, nseg, need);
        } else {
            const size_t cap = workspace && workspace_bytes > kCounterBytes ? workspace_bytes - kCounterBytes : 0;
            nseg = kda::seq_split_auto(B, T, H, (int)dk, (int)dv, is_bf16, rerun, layout, cap);
            if (nseg >= 2) split_ws = static_cast<char *>(workspace) + kCounterBytes;
        }
    }
    const int wide = kda::seq_layout(B, T, H, (int)dk, (int)dv, is_bf16, rerun, nseg, layout);
    // the library's two-segment split, guarded against gates that keep
    // memory when one pass would then be faster
    int guarded = 0, fallback_wide = 0;
    if (req_seg == 0 && !rerun && split_ws) {
        fallback_wide = kda::seq_layout(B, T, H, (int)dk, (int)dv, is_bf16, 0, 1, layout);
        guarded = kda::seq_split_guarded(B, T, H, (int)dk, (int)dv, is_bf16, nseg, wide, fallback_wide) ? 1 : 0;
    }
    hipError_t e = kda::launch_chunk_fwd(q, k, v, g, beta, initial_state, final_state, o, B, T, H,
                                         (int)dk, (int)dv, is_bf16, nseg, split_ws, slots, n_slots,
                                         pairwise ? 1 : 0, cu_seqlens, fused ? z : nullptr,
                                         fused ? Ag : nullptr, rerun, wide, guarded, fallback_wide, s);
    if (e != hipSuccess) return hip_fail(e, "kda_chunk_fwd launch");
    return ok();
}

}  // namespace

namespace kda {

// The shared prefill implementation and the error report, for the entry
// point of kda_noalloc.hip (its own source file holds its device array).
int chunk_fwd_entry(const char *who, const void *q, const void *k, const void *v, const float *g,
                    const void *beta, const float *initial_state, float *final_state, void *o,
                    void *workspace, size_t workspace_bytes, int64_t B, int64_t T, int64_t H,
                    int64_t dk, int64_t dv, int dtype, unsigned flags, const void *z,
                    const float *Ag, void *stream) {
    return chunk_fwd_impl(who, q, k, v, g, beta, initial_state, final_state, o, workspace,
                          workspace_bytes, B, T, H, dk, dv, dtype, flags, nullptr, 0, nullptr, z,
                          Ag, stream);
}

int report_error(int code, const char *msg) { return fail(code, "%s", msg); }

}  // namespace kda

extern "C" {

int kda_chunk_fwd(const void *q, const void *k, const void *v, const float *g, const void *beta,
                  const float *initial_state, float *final_state, void *o, void *workspace,
                  size_t workspace_bytes, int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                  int dtype, unsigned flags, void *stream) {
    return chunk_fwd_impl("kda_chunk_fwd", q, k, v, g, beta, initial_state, final_state, o,
                          workspace, workspace_bytes, B, T, H, dk, dv, dtype, flags, nullptr, 0,
                          nullptr, nullptr, nullptr, stream);
}

int kda_chunk_fwd_gated(const void *q, const void *k, const void *v, const void *z, const float *A,
                        const void *beta, const float *initial_state, float *final_state, void *o,
                        void *workspace, size_t workspace_bytes, int64_t B, int64_t T, int64_t H,
                        int64_t dk, int64_t dv, int dtype, unsigned flags, void *stream) {
    if (!z || !A)
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_chunk_fwd_gated: null pointer (z and A are required)");
    return chunk_fwd_impl("kda_chunk_fwd_gated", q, k, v, nullptr, beta, initial_state, final_state, o,
                          workspace, workspace_bytes, B, T, H, dk, dv, dtype, flags, nullptr, 0,
                          nullptr, z, A, stream);
}

int kda_chunk_fwd_pooled(const void *q, const void *k, const void *v, const float *g,
                         const void *beta, float *state_pool, const int32_t *slots, void *o,
                         void *workspace, size_t workspace_bytes, int64_t B, int64_t T,
                         int64_t n_slots, int64_t H, int64_t dk, int64_t dv, int dtype,
                         unsigned flags, void *stream) {
    if (!state_pool || !slots)
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_chunk_fwd_pooled: null state_pool or slots");
    if (n_slots <= 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_chunk_fwd_pooled: n_slots must be positive");
    int64_t np = n_slots;
    if (!mul_ok(np, H) || !mul_ok(np, dk) || !mul_ok(np, dv))
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_chunk_fwd_pooled: pool size overflows");
    if (reinterpret_cast<uintptr_t>(slots) & 3u)
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_chunk_fwd_pooled: slots must be 4-byte aligned");
    if (static_cast<const void *>(slots) == o || static_cast<const void *>(state_pool) == o)
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_chunk_fwd_pooled: o must not alias an input");
    return chunk_fwd_impl("kda_chunk_fwd_pooled", q, k, v, g, beta, state_pool, state_pool, o,
                          workspace, workspace_bytes, B, T, H, dk, dv, dtype, flags, slots,
                          n_slots, nullptr, nullptr, nullptr, stream);
}

}  // extern "C"

// kda_chunk_fwd_varlen_pooled and its fused-gate form (z, A instead of g)
static int varlen_pooled_impl(const char *who, const void *q, const void *k, const void *v,
                              const float *g, const void *z, const float *A, const void *beta,
                              float *state_pool, const int32_t *slots, const int64_t *cu_seqlens,
                              void *o, int64_t B, int64_t total_tokens, int64_t n_slots, int64_t H,
                              int64_t dk, int64_t dv, int dtype, unsigned flags, void *stream) {
    if (!cu_seqlens) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: null cu_seqlens", who);
    if (reinterpret_cast<uintptr_t>(cu_seqlens) & 7u)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: cu_seqlens must be 8-byte aligned", who);
    if (!kda::seq_split_supported((int)dk, (int)dv, dtype == KDA_BF16))
        return fail(KDA_ERR_UNSUPPORTED, "%s: needs bf16 inputs, dk = 128, dv in {64, 128}", who);
    if (flags & (KDA_FLAG_CHECK_RANGE | KDA_FLAG_SEGMENTS_MASK))
        return fail(KDA_ERR_INVALID_ARGUMENT,
                    "%s: the range check and the sequence split take the [B, T, H] layout", who);
    if (int e = check_pool(who, state_pool, slots, n_slots, H, dk, dv)) return e;
    if (static_cast<const void *>(slots) == o || static_cast<const void *>(state_pool) == o ||
        static_cast<const void *>(cu_seqlens) == o)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: o must not alias an input", who);
    // one pass (no split), the packed tokens as T of a single batch row for
    // the size checks; the kernel reads sequence b's rows from cu_seqlens
    return chunk_fwd_impl(who, q, k, v, g, beta, state_pool, state_pool, o, nullptr, 0, B,
                          total_tokens, H, dk, dv, dtype, flags | KDA_FLAG_SEGMENTS(1), slots,
                          n_slots, cu_seqlens, z, A, stream);
}

extern "C" {

int kda_chunk_fwd_varlen_pooled(const void *q, const void *k, const void *v, const float *g,
                                const void *beta, float *state_pool, const int32_t *slots,
                                const int64_t *cu_seqlens, void *o, int64_t B,
                                int64_t total_tokens, int64_t n_slots, int64_t H, int64_t dk,
                                int64_t dv, int dtype, unsigned flags, void *stream) {
    return varlen_pooled_impl("kda_chunk_fwd_varlen_pooled", q, k, v, g, nullptr, nullptr, beta,
                              state_pool, slots, cu_seqlens, o, B, total_tokens, n_slots, H, dk,
                              dv, dtype, flags, stream);
}

int kda_chunk_fwd_varlen_pooled_gated(const void *q, const void *k, const void *v, const void *z,
                                      const float *A, const void *beta, float *state_pool,
                                      const int32_t *slots, const int64_t *cu_seqlens, void *o,
                                      int64_t B, int64_t total_tokens, int64_t n_slots, int64_t H,
                                      int64_t dk, int64_t dv, int dtype, unsigned flags,
                                      void *stream) {
    const char *who = "kda_chunk_fwd_varlen_pooled_gated";
    if (!z || !A) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: null pointer (z and A are required)", who);
    return varlen_pooled_impl(who, q, k, v, nullptr, z, A, beta, state_pool, slots, cu_seqlens, o,
                              B, total_tokens, n_slots, H, dk, dv, dtype, flags, stream);
}

}  // extern "C"

namespace {

int decode_step_impl(const void *q, const void *k, const void *v, const void *z, const float *A,
                     const void *beta, float *state, void *o, int64_t N, int64_t H, int64_t dk,
                     int64_t dv, int dtype, const int32_t *slots, int64_t n_slots, void *stream) {
    if (int e = check_dtype(dtype)) return e;
    if (!q || !k || !v || !z || !A || !beta || !state || !o)
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_decode_step: null pointer");
    if (N <= 0 || H <= 0 || dk <= 0 || dv <= 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_decode_step: sizes must be positive");
    if (!valid_dim(dk) || !valid_dim(dv))
        return fail(KDA_ERR_UNSUPPORTED, "kda_decode_step: dk=%lld dv=%lld must be in {32,64,128}",
                    (long long)dk, (long long)dv);
    int64_t ns = N;
    if (!mul_ok(ns, H) || !mul_ok(ns, dk) || !mul_ok(ns, dv))
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_decode_step: element count overflows");
    if (N * H > 0x7fffffffLL)
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_decode_step: N*H too large");
    const void *ptrs[] = {q, k, v, z, A, beta, state, o};
    for (const void *p : ptrs)
        if (!aligned16(p))
            return fail(KDA_ERR_INVALID_ARGUMENT, "kda_decode_step: pointers must be 16-byte aligned");
    const void *ins[] = {q, k, v, z, A, beta, state};
    for (const void *p : ins)
        if (p == o) return fail(KDA_ERR_INVALID_ARGUMENT, "kda_decode_step: o must not alias an input");
    hipError_t e = kda::launch_decode_step(q, k, v, z, A, beta, state, o, N, H, (int)dk, (int)dv,
                                           dtype == KDA_BF16, slots, n_slots,
                                           static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "kda_decode_step launch");
    return ok();
}

}  // namespace

extern "C" {

size_t kda_chunk_bwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                    int dtype) {
    if (B <= 0 || T <= 0 || H <= 0 || !valid_dim(dk) || !valid_dim(dv)) return 0;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return 0;
    int64_t n = B;
    if (!mul_ok(n, T) || !mul_ok(n, H) || !mul_ok(n, dk) || !mul_ok(n, dv)) return 0;
    // the range-check counter, then the larger of the two paths' buffers
    const size_t tok = kda::bwd_workspace_bytes(B, T, H, (int)dk, (int)dv);
    const size_t chk = kda::cbwd_workspace_bytes(B, T, H, (int)dk, (int)dv);
    return kCounterBytes + (tok > chk ? tok : chk);
}

size_t kda_chunk_bwd_workspace_size_flags(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                          int dtype, unsigned flags, int64_t segment_tokens) {
    if (B <= 0 || T <= 0 || H <= 0 || !valid_dim(dk) || !valid_dim(dv)) return 0;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return 0;
    if (segment_tokens < 0 && segment_tokens != KDA_BWD_SEGMENTS_MIN_WORKSPACE) return 0;
    int64_t n = B;
    if (!mul_ok(n, T) || !mul_ok(n, H) || !mul_ok(n, dk) || !mul_ok(n, dv)) return 0;
    if (flags & KDA_FLAG_TOKEN_BACKWARD)
        return kCounterBytes + kda::bwd_workspace_bytes(B, T, H, (int)dk, (int)dv);
    if (segment_tokens == KDA_BWD_SEGMENTS_MIN_WORKSPACE)
        return kCounterBytes + kda::cbwd_min_workspace_bytes(B, T, H, (int)dk, (int)dv);
    const int64_t seg = segment_tokens == 0 ? T : (segment_tokens + 31) / 32 * 32;
    return kCounterBytes + kda::cbwd_workspace_bytes_seg(B, T, H, (int)dk, (int)dv, seg);
}

int kda_chunk_bwd(const void *q, const void *k, const void *v, const float *g, const void *beta,
                  const float *initial_state, const void *d_o, const float *d_final_state,
                  float *dq, float *dk, float *dv, float *dg, float *dbeta,
                  float *d_initial_state, void *workspace, size_t workspace_bytes, int64_t B,
                  int64_t T, int64_t H, int64_t dk_dim, int64_t dv_dim, int dtype, unsigned flags,
                  void *stream) {
    const char *who = "kda_chunk_bwd";
    if (int e = check_dtype(dtype)) return e;
    if (flags & ~unsigned(KDA_FLAG_CHECK_RANGE | KDA_FLAG_TOKEN_BACKWARD))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown flag bits 0x%x", who, flags);
    const bool token = (flags & KDA_FLAG_TOKEN_BACKWARD) != 0;
    if (token && (flags & KDA_FLAG_CHECK_RANGE))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: the token-level path assumes no decay range to check", who);
    if (!q || !k || !v || !g || !beta || !d_o || !dq || !dk || !dv || !dg || !dbeta || !workspace)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: null pointer (all but initial_state, "
                    "d_final_state and d_initial_state are required)", who);
    if (B <= 0 || T <= 0 || H <= 0 || dk_dim <= 0 || dv_dim <= 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: sizes must be positive", who);
    if (!valid_dim(dk_dim) || !valid_dim(dv_dim))
        return fail(KDA_ERR_UNSUPPORTED, "%s: dk=%lld dv=%lld must be in {32,64,128}", who,
                    (long long)dk_dim, (long long)dv_dim);
    int64_t n = B;
    if (!mul_ok(n, T) || !mul_ok(n, H) || !mul_ok(n, dk_dim) || !mul_ok(n, dv_dim))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: element count overflows", who);
    if (B * H > 0x7fffffffLL) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: B*H too large", who);
    // the token path needs its whole-sequence buffers; the chunked path runs
    // in the longest segments the workspace holds (at least 32 tokens)
    const size_t need = kda_chunk_bwd_workspace_size_flags(B, T, H, dk_dim, dv_dim, dtype, flags,
                                                           token ? 0 : KDA_BWD_SEGMENTS_MIN_WORKSPACE);
    if (workspace_bytes < need)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: needs a workspace of at least %zu bytes", who, need);
    const void *ptrs[] = {q, k, v, g, beta, initial_state, d_o, d_final_state, dq, dk, dv, dg,
                          dbeta, d_initial_state, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: pointers must be 16-byte aligned", who);
    const void *outs[] = {dq, dk, dv, dg, dbeta, d_initial_state, workspace};
    const void *ins[] = {q, k, v, g, beta, initial_state, d_o, d_final_state};
    for (const void *po : outs)
        for (const void *pi : ins)
            if (po && po == pi)
                return fail(KDA_ERR_INVALID_ARGUMENT, "%s: outputs must not alias inputs", who);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (flags & KDA_FLAG_CHECK_RANGE) {
        unsigned int *bad = static_cast<unsigned int *>(workspace);
        hipError_t e = hipMemsetAsync(bad, 0, sizeof(unsigned int), s);
        if (e != hipSuccess) return hip_fail(e, "kda_chunk_bwd range check memset");
        e = kda::launch_range_check(g, B, T, H, dk_dim, bad, s);
        if (e != hipSuccess) return hip_fail(e, "kda_chunk_bwd range check launch");
        unsigned int nbad = 0;
        e = hipMemcpyAsync(&nbad, bad, sizeof nbad, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_fail(e, "kda_chunk_bwd range check readback");
        if (nbad)
            return fail(KDA_ERR_RANGE, "%s: %u gate values or 16-token tile sums outside [-5,0] / [-80,0]", who,
                        nbad);
    }
    float *ws = reinterpret_cast<float *>(static_cast<char *>(workspace) + kCounterBytes);
    hipError_t e =
        token ? kda::launch_chunk_bwd(q, k, v, g, beta, initial_state, d_o, d_final_state, dq, dk, dv,
                                      dg, dbeta, d_initial_state, ws, B, T, H, (int)dk_dim,
                                      (int)dv_dim, dtype == KDA_BF16, s)
              : kda::launch_chunk_bwd_chunked(q, k, v, g, beta, initial_state, d_o, d_final_state, dq,
                                              dk, dv, dg, dbeta, d_initial_state, ws,
                                              workspace_bytes - kCounterBytes, B, T, H,
                                              (int)dk_dim, (int)dv_dim, dtype == KDA_BF16, s);
    if (e != hipSuccess) return hip_fail(e, "kda_chunk_bwd launch");
    return ok();
}

int kda_decode_step(const void *q, const void *k, const void *v, const void *z, const float *A,
                    const void *beta, float *state, void *o, int64_t N, int64_t H, int64_t dk,
                    int64_t dv, int dtype, void *stream) {
    return decode_step_impl(q, k, v, z, A, beta, state, o, N, H, dk, dv, dtype, nullptr, 0, stream);
}

int kda_decode_step_pooled(const void *q, const void *k, const void *v, const void *z,
                           const float *A, const void *beta, float *state_pool,
                           const int32_t *slots, void *o, int64_t N, int64_t n_slots, int64_t H,
                           int64_t dk, int64_t dv, int dtype, void *stream) {
    if (int e = check_pool("kda_decode_step_pooled", state_pool, slots, n_slots, H, dk, dv)) return e;
    if (static_cast<const void *>(slots) == o)
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_decode_step_pooled: o must not alias an input");
    return decode_step_impl(q, k, v, z, A, beta, state_pool, o, N, H, dk, dv, dtype, slots, n_slots,
                            stream);
}

int kda_state_pool_reset(float *state_pool, const int32_t *slots, int64_t n, int64_t n_slots,
                         int64_t H, int64_t dk, int64_t dv, void *stream) {
    if (int e = check_pool("kda_state_pool_reset", state_pool, slots, n_slots, H, dk, dv)) return e;
    if (n <= 0) return fail(KDA_ERR_INVALID_ARGUMENT, "kda_state_pool_reset: n must be positive");
    if (n > 0x7fffffffLL) return fail(KDA_ERR_INVALID_ARGUMENT, "kda_state_pool_reset: n too large");
    hipError_t e = kda::launch_pool_reset(state_pool, slots, n, n_slots, H * dk * dv,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "kda_state_pool_reset launch");
    return ok();
}

}  // extern "C"
