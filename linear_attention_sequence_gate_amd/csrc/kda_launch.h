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
// nseg >= 2 splits each sequence into that many segments (pipelined path
// only; split_ws must hold seq_split_workspace() bytes), else one pass.
// slots != nullptr: S0 and ST index a state pool [n_slots, H, dk, dv] by
// slots[b] (sequences whose slot lies outside the pool are skipped).
// pairwise: the diagonal 16-token tiles by position pairs (pipelined path).
// cu_seqlens != nullptr: variable-length sequences packed along the token
// axis (pipelined path, one pass; T is then the packed token count).
// z != nullptr: the gate is evaluated inside the kernel from z (input dtype,
// laid out like k) and the [H, dk] table Ag; g is not read (pipelined path).
// wide: one workgroup per chain (pipelined path, dv = 128, not pairwise).
// guarded (two segments, stopping split): a probe of the second segment's
// transitions picks on the device between the split and one pass in the
// fallback_wide layout.
hipError_t launch_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                            const void *beta, const float *S0, float *ST, void *o, int64_t B,
                            int64_t T, int64_t H, int dk, int dv, int is_bf16, int nseg,
                            void *split_ws, const int *slots, int64_t n_slots, int pairwise,
                            const int64_t *cu_seqlens, const void *z, const float *Ag,
                            int split_rerun, int wide, int guarded, int fallback_wide,
                            hipStream_t s);

// Sequence split of the pipelined chunk path (bf16, dk = 128, dv in {64, 128}).
bool seq_split_supported(int dk, int dv, int is_bf16);
// Segment length for nseg segments (a multiple of the 32-token chunk) and the
// number of segments that length gives.
int64_t seq_split_segment_len(int64_t T, int nseg);
int seq_split_effective(int64_t T, int nseg);
// Segment count picked for these sizes (1 = no split), for the stopping
// split or (rerun) the one whose last phase reruns whole segments, over the
// workgroup layouts allowed (layout: -1 either, 0 per 64-column slice, 1 per
// chain) and the counts whose buffers fit in ws_cap bytes.
int seq_split_auto(int64_t B, int64_t T, int64_t H, int dk, int dv, int is_bf16, int rerun,
                   int layout, size_t ws_cap = SIZE_MAX);
// One workgroup per chain: bf16, dk = dv = 128.
bool seq_wide_supported(int dk, int dv, int is_bf16);
// The layout (0 per slice, 1 per chain) for P segments: `layout` when it is
// forced (>= 0), else the cheaper one in the same model.
int seq_layout(int64_t B, int64_t T, int64_t H, int dk, int dv, int is_bf16, int rerun, int P,
               int layout);
// Whether a two-segment stopping split in layout `wide` is guarded against
// gates that keep memory (its worst case is slower than one pass in
// fallback_wide), P the requested count.
bool seq_split_guarded(int64_t B, int64_t T, int64_t H, int dk, int dv, int is_bf16, int P,
                       int wide, int fallback_wide);
// Device bytes the split needs (0 when it does not split).
size_t seq_split_workspace(int64_t B, int64_t T, int64_t H, int dk, int dv, int nseg);

bool chunk_fwd_supported(int dk, int dv, int is_bf16);
// Prefill of the shapes chunk_fwd_supported leaves out (fp32 inputs at dk =
// 128): the reverse mode's chunk preparation and forward pass with outputs,
// in fp32 arithmetic; it needs cb_prefill_workspace_bytes of workspace.
// With slots, the states are rows of a pool as in the pooled calls.
size_t cb_prefill_workspace_bytes(int64_t B, int64_t T, int64_t H, int dk);
hipError_t launch_chunk_fwd_cb(const void *q, const void *k, const void *v, const float *g,
                               const void *beta, const float *S0, float *ST, void *o, void *ws,
                               size_t ws_bytes, int64_t B, int64_t T, int64_t H, int dk, int dv,
                               int is_bf16, const int *slots, int64_t n_slots, hipStream_t s);

// slots == nullptr: state is [N, H, dk, dv]; else state is a pool
// [n_slots, H, dk, dv] and sequence n uses slot slots[n] (heads of a slot
// outside the pool are skipped).
hipError_t launch_decode_step(const void *q, const void *k, const void *v, const void *z,
                              const float *A, const void *beta, float *state, void *o,
                              int64_t N, int64_t H, int dk, int dv, int is_bf16, const int *slots,
                              int64_t n_slots, hipStream_t s);

// Zero the listed slots of a state pool; per_slot = H * dk * dv floats.
hipError_t launch_pool_reset(float *pool, const int *slots, int64_t n, int64_t n_slots,
                             int64_t per_slot, hipStream_t s);

// Reverse mode of the gate: dz and dA from dg over `rows` rows of H*dk
// columns; `part` holds gate_bwd_workspace_bytes() of per-row-range dA shares.
hipError_t launch_gate_bwd(const void *z, const float *A, const float *dg, float *dz, float *dA,
                           float *part, int64_t rows, int H, int dk, int is_bf16, hipStream_t s);
size_t gate_bwd_workspace_bytes(int64_t rows, int C);

// Reverse mode of the recurrence (token by token over 32-column slices,
// states recomputed from checkpoints every 8 tokens; `ckpt` is the
// workspace, bwd_workspace_bytes() long).  Gradients are fp32; dST and dS0
// may be null.
hipError_t launch_chunk_bwd(const void *q, const void *k, const void *v, const float *g,
                            const void *beta, const float *S0, const void *dout, const float *dST,
                            float *dq, float *dk, float *dv, float *dg, float *dbeta, float *dS0,
                            float *ckpt, int64_t B, int64_t T, int64_t H, int dk_, int dv_,
                            int is_bf16, hipStream_t s);
size_t bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int dk, int dv);

// Reverse mode in 16-token chunks on the fp32 matrix cores (the gate floor's
// decay range assumed: every 16-token sum of g from the sequence start is
// >= -80).  `ws` holds ws_bytes: cbwd_workspace_bytes() runs the sequence in
// one segment; less runs it in the longest segments that fit
// (cbwd_segment_tokens; hipErrorInvalidValue below 32 tokens).
hipError_t launch_chunk_bwd_chunked(const void *q, const void *k, const void *v, const float *g,
                                    const void *beta, const float *S0, const void *dout,
                                    const float *dST, float *dq, float *dk, float *dv, float *dg,
                                    float *dbeta, float *dS0, float *ws, size_t ws_bytes, int64_t B,
                                    int64_t T, int64_t H, int dk_, int dv_, int is_bf16,
                                    hipStream_t s);
size_t cbwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int dk, int dv);
// Segments of `seg` tokens (a multiple of 32; >= T: one segment).
size_t cbwd_workspace_bytes_seg(int64_t B, int64_t T, int64_t H, int dk, int dv, int64_t seg);
int64_t cbwd_segment_tokens(int64_t B, int64_t T, int64_t H, int dk, int dv, size_t bytes);
// The smallest workspace over every segment length (the whole sequence included).
size_t cbwd_min_workspace_bytes(int64_t B, int64_t T, int64_t H, int dk, int dv);

// The C ABI's shared chunked-prefill implementation (validation, the gate
// staging of unfused shapes, the sequence split, the launches) with a caller's
// workspace, and the error report behind kda_last_error(); defined in
// kda_api.cpp.
int chunk_fwd_entry(const char *who, const void *q, const void *k, const void *v, const float *g,
                    const void *beta, const float *initial_state, float *final_state, void *o,
                    void *workspace, size_t workspace_bytes, int64_t B, int64_t T, int64_t H,
                    int64_t dk, int64_t dv, int dtype, unsigned flags, const void *z,
                    const float *Ag, void *stream);
int report_error(int code, const char *msg);

}  // namespace kda
