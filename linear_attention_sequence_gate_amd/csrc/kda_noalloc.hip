// kda_chunk_fwd_gated_noalloc: the gated chunkwise prefill for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  Its workspace -- the sequence
// split's per-segment states and transitions, or the staged g of shapes
// without the fused gate -- is the fixed device array below, one copy per
// GPU at that GPU's own address.  Nothing here allocates or frees device
// memory.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "kda.h"
#include "kda_launch.h"

static_assert(KDA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");

// The scratch array.  Host code never uses this name as an address (on the
// host it is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, per device, below.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch_ptr[kMaxDevices];    // device address of `scratch` on each device

int hip_error(hipError_t e, const char *what) {
    char buf[256];
    snprintf(buf, sizeof buf, "kda_chunk_fwd_gated_noalloc: %s: %s", what, hipGetErrorString(e));
    return kda::report_error(KDA_ERR_HIP, buf);
}

// The scratch address on the device the stream belongs to, looked up once per
// device with that device current.
int scratch_for_stream(hipStream_t s, void **out) {
    int dev = -1;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return hip_error(e, "device of the stream");
    if (dev < 0 || dev >= kMaxDevices)
        return kda::report_error(KDA_ERR_UNSUPPORTED,
                                 "kda_chunk_fwd_gated_noalloc: device index beyond 63");
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return hip_error(e, "current device");
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_error(e, "select device");
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return hip_error(e, "scratch address");
        if (e2 != hipSuccess) return hip_error(e2, "restore device");
        if (!p) return kda::report_error(KDA_ERR_HIP, "kda_chunk_fwd_gated_noalloc: null scratch address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KDA_OK;
}

}  // namespace

extern "C" int kda_chunk_fwd_gated_noalloc(const void *q, const void *k, const void *v, const void *z,
                                           const float *A, const void *beta,
                                           const float *initial_state, float *final_state, void *o,
                                           int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                           int dtype, unsigned flags, void *stream) {
    const char *who = "kda_chunk_fwd_gated_noalloc";
    if (!z || !A)
        return kda::report_error(KDA_ERR_INVALID_ARGUMENT,
                                 "kda_chunk_fwd_gated_noalloc: null pointer (z and A are required)");
    // what the call would need from a workspace: an explicit segment count
    // (or the staged g of an unfused shape) beyond the array is an error; the
    // automatic count falls back to one pass when its buffers do not fit
    const int req_seg = (int)((flags & KDA_FLAG_SEGMENTS_MASK) >> KDA_FLAG_SEGMENTS_SHIFT);
    size_t need = kda_chunk_fwd_gated_workspace_size(B, T, H, dk, dv, dtype);
    if (req_seg >= 2 && need != 0) {
        const size_t seg = kda_chunk_fwd_workspace_size_segments(B, T, H, dk, dv, dtype, req_seg);
        const size_t one = kda_chunk_fwd_workspace_size(B, T, H, dk, dv, dtype);
        need = seg == 0 ? 0 : need - one + seg;
    } else if (need != 0) {
        // the automatic split takes no scratch when it does not fit: count
        // only the staged g (unfused shapes) and the 256-byte counter
        const size_t one = kda_chunk_fwd_workspace_size_segments(B, T, H, dk, dv, dtype, 1);
        const size_t full = kda_chunk_fwd_workspace_size(B, T, H, dk, dv, dtype);
        if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES) need = need - full + one;
    }
    if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES) {
        char buf[256];
        snprintf(buf, sizeof buf,
                 "%s: these sizes need %zu bytes of scratch; the library's fixed scratch holds %u "
                 "bytes (use kda_chunk_fwd_gated with a workspace)",
                 who, need, (unsigned)KDA_NOALLOC_SCRATCH_BYTES);
        return kda::report_error(KDA_ERR_INVALID_ARGUMENT, buf);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    void *ws = nullptr;
    if (int e = scratch_for_stream(s, &ws)) return e;
    return kda::chunk_fwd_entry(who, q, k, v, nullptr, beta, initial_state, final_state, o, ws,
                                KDA_NOALLOC_SCRATCH_BYTES, B, T, H, dk, dv, dtype, flags, z, A,
                                stream);
}
