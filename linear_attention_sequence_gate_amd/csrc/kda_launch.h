// Host-side launchers, one per kernel family.  Arguments are validated by the
// C ABI layer (kda_api.cpp) before any of these is called.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace kda {

hipError_t launch_gate(const void *z, const float *A, float *g, int64_t n_elems, int H, int dk,
                       int is_bf16, hipStream_t s);

hipError_t launch_range_check(const float *g, int64_t B, int64_t T, int64_t H, int64_t dk,
                              unsigned int *bad, hipStream_t s);

// Returns hipErrorInvalidValue when no kernel instance exists for (dk, dtype).
hipError_t launch_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                            const void *beta, const float *S0, float *ST, void *o, int64_t B,
                            int64_t T, int64_t H, int dk, int dv, int is_bf16, hipStream_t s);

bool chunk_fwd_supported(int dk, int dv, int is_bf16);

hipError_t launch_decode_step(const void *q, const void *k, const void *v, const void *z,
                              const float *A, const void *beta, float *state, void *o,
                              int64_t N, int64_t H, int dk, int dv, int is_bf16, hipStream_t s);

}  // namespace kda
