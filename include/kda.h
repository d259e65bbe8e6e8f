/*
 * libkda -- Kimi Delta Attention (KDA) forward hot path for AMD MI355X (gfx950).
 *
 * KDA is a recurrent linear attention whose fixed-size per-head state
 * S in R^{dk x dv} replaces a growing KV cache ("Kimi K3 internal structure
 * analysis", section "Sequence mixing: 3 KDA layers per global MLA layer";
 * the studioglobal.ai summary of the Kimi K3 report, section on KDA: memory
 * and decoding work stay fixed as the context grows).  Per token t:
 *
 *     g_t   = -5 * sigmoid(exp(A) * z_t)            (gate, floor gmin = -5)
 *     S'    = Diag(exp(g_t)) S_{t-1}                (channel-wise retention, first)
 *     u_t   = beta_t (v_t - S'^T k_t)
 *     S_t   = S' + k_t u_t^T                        (delta-rule write)
 *     o_t   = S_t^T q_t
 *
 * Every entry point takes the state in and hands the state out, so a sequence
 * can be cut anywhere and resumed (the page's "Infrastructure for a 3T-class
 * MoE" section: a segment acts on its incoming state and emits a state).
 *
 * Conventions shared by all calls
 * -------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller, contiguous
 *    row-major in the layouts stated per call, with 16-byte aligned bases.
 *    The library never allocates or frees device memory.  Its one piece of
 *    device state is the fixed scratch array of kda_chunk_fwd_gated_noalloc.
 *  - `dtype` selects the element type of q, k, v, z, beta and o:
 *    KDA_F32 (IEEE fp32) or KDA_BF16 (bfloat16).  A, g and the state are fp32.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *    work on it and return; faults inside kernels surface at the caller's
 *    next synchronisation with that stream, as usual in HIP.
 *  - Return value: KDA_OK or a negative error code.  Host-side validation runs
 *    before any HIP call, so an invalid call touches no device memory.
 *    kda_last_error() describes the most recent failure of the calling thread.
 *  - Sizes: B, T, H, N >= 1; dk, dv in {32, 64, 128}, every combination and
 *    both dtypes.  fp32 inputs at dk = 128 in the prefill calls (a 64-token
 *    fp32 tile set that wide exceeds the 160 KiB of LDS) run 16-token chunks
 *    through device buffers instead: they need a workspace (also in the
 *    pooled call), and the packed call returns UNSUPPORTED for them.
 *    Index-width limits (INVALID_ARGUMENT beyond them): kda_gate H*dk <= 2^28;
 *    kda_chunk_fwd B*H <= 2^24 and H*max(dk,dv)*256 < 2^32; kda_decode_step
 *    N*H < 2^31.
 *  - No scaling or normalisation is applied to q or k; that is the caller's.
 *  - Concurrent calls that share an output buffer race.  Apart from
 *    kda_chunk_fwd_gated_noalloc's scratch array (calls of it that overlap on
 *    one GPU race), the library keeps no global state of its own.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = -1, /* null pointer, size <= 0, overflow, misalignment, small workspace */
    KDA_ERR_UNSUPPORTED = -2,      /* dk/dv outside {32,64,128}, unknown dtype, a shape a path does not take */
    KDA_ERR_HIP = -3,              /* a HIP runtime call or kernel launch failed */
    KDA_ERR_RANGE = -4             /* KDA_FLAG_CHECK_RANGE found g outside [-5, 0] or a 16-token sum < -80 */
};

/* Flags for kda_chunk_fwd (and, where noted, kda_chunk_bwd). */
enum {
    /* Before the forward pass, check on the device that every g lies in
     * [-5, 0] and every 16-token tile sum (tiles aligned to token 0 of the
     * call) lies in [-80, 0] -- the range the gate's floor guarantees and the
     * chunked kernel relies on.  Synchronises the stream; debugging only. */
    KDA_FLAG_CHECK_RANGE = 1u,
    /* Compute the diagonal 16-token tiles of A and P by position pairs,
     * sum_c x_rc k_sc 2^(lam_rc - lam_sc) with the log-decay lam kept in log
     * space, instead of dense MFMA tiles of decay-scaled operands.  This is
     * the path the gate floor made unnecessary ("Kimi K3 internal structure
     * analysis", section "Sequence mixing: 3 KDA layers per global MLA
     * layer": without a floor the reciprocal cumulative decay inside a
     * diagonal tile can overflow).  With it, g may lie anywhere <= 0 (no
     * 16-token range bound).  bf16, dk = 128, dv in {64, 128}; slower. */
    KDA_FLAG_PAIRWISE_DIAGONAL = 2u,
    /* Bits 8..15: segments per sequence for the sequence-parallel path
     * (bf16, dk = 128, dv in {64, 128}): 0 = chosen by the library, 1 = never
     * split, n >= 2 = split into n segments (the count a 32-token-aligned
     * segment length gives).  See kda_chunk_fwd. */
    KDA_FLAG_SEGMENTS_SHIFT = 8,
    KDA_FLAG_SEGMENTS_MASK = 0xff00u,
    /* kda_chunk_bwd only: take the token-level reverse mode, which assumes
     * nothing about the decay range (any g <= 0), instead of the chunked one.
     * Slower. */
    KDA_FLAG_TOKEN_BACKWARD = 0x10000u,
    /* Sequence split: rerun every segment after the first in full in the
     * last phase, instead of only its chunks up to the point where the
     * segment's transition became exactly zero (see kda_chunk_fwd).  Faster
     * when the gates keep memory over more than about half a segment; the
     * segment count is then chosen for this scheme. */
    KDA_FLAG_SPLIT_FULL_RERUN = 0x20000u,
    /* Workgroup layout of the pipelined chunk path at dv = 128 (bf16,
     * dk = 128): one workgroup per chain covering all 128 state columns, so
     * each chunk's decayed operands and scores are formed once per chain,
     * or one per 64-column slice (two per chain, each forming them itself:
     * twice the chips' compute units filled by as many chains).  Without
     * either flag the library picks, with the segment count; with one it
     * takes that layout (PER_CHAIN is rejected for other shapes and with
     * KDA_FLAG_PAIRWISE_DIAGONAL).  Results agree to rounding order: each
     * state column's arithmetic is the same, only which workgroup runs it
     * differs. */
    KDA_FLAG_WORKGROUP_PER_CHAIN = 0x40000u,
    KDA_FLAG_WORKGROUP_PER_SLICE = 0x80000u
};
#define KDA_FLAG_SEGMENTS(n) ((unsigned)(n) << KDA_FLAG_SEGMENTS_SHIFT)

/*
 * kda_gate -- the K3 gate, g = -5 * sigmoid(exp(A[h,c]) * z[b,t,h,c]).
 *   ("Kimi K3 internal structure analysis", section "Sequence mixing: 3 KDA
 *   layers per global MLA layer": the retention parameterisation with g_min = -5.)
 *   z : [B, T, H, dk]  dtype            (input)
 *   A : [H, dk]        fp32             (input)
 *   g : [B, T, H, dk]  fp32             (output; may not alias z)
 * The result lies in [-5, 0]; alpha = exp(g) is the per-channel retention.
 */
int kda_gate(const void *z, const float *A, float *g,
             int64_t B, int64_t T, int64_t H, int64_t dk,
             int dtype, void *stream);

/*
 * kda_gate_bwd -- reverse mode of kda_gate: the gradients of L = <g, dg>
 * with respect to z and A.  The gate is the one of "Kimi K3 internal
 * structure analysis", section "Sequence mixing: 3 KDA layers per global MLA
 * layer"; the pages say nothing of training, so the reverse mode is derived
 * from it.  With x = exp(A) z:
 *   dz = -5 sigmoid'(x) exp(A) dg,   dA[h,c] = sum over (b,t) of -5 sigmoid'(x) x dg
 *   z  : [B, T, H, dk] dtype   (input, as given to kda_gate)
 *   A  : [H, dk]       fp32    (input)
 *   dg : [B, T, H, dk] fp32    (input, e.g. kda_chunk_bwd's dg)
 *   dz : [B, T, H, dk] fp32    (output)
 *   dA : [H, dk]       fp32    (output, overwritten)
 *   workspace : kda_gate_bwd_workspace_size() bytes (per-row-range shares of
 *               dA, added in a fixed order: the result does not depend on
 *               scheduling)
 * Outputs must not alias inputs or each other.
 */
size_t kda_gate_bwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t dk);
int kda_gate_bwd(const void *z, const float *A, const float *dg, float *dz, float *dA,
                 void *workspace, size_t workspace_bytes, int64_t B, int64_t T, int64_t H,
                 int64_t dk, int dtype, void *stream);

/*
 * Workspace bytes kda_chunk_fwd needs for these sizes with the segment count
 * the library picks (flags without segment bits): 256 bytes for the
 * range-check counter, plus, when the sizes take the sequence-parallel path,
 * its per-segment states and transitions (fp32: (P-1) B H dk dv for the
 * segments' initial states, (P-2) B H (dk dv + dk dk) for the middle
 * segments' zero-start states and transition matrices, P segments).
 * Returns 0 for invalid sizes.
 */
size_t kda_chunk_fwd_workspace_size(int64_t B, int64_t T, int64_t H,
                                    int64_t dk, int64_t dv, int dtype);

/*
 * Segments per sequence kda_chunk_fwd uses for these sizes when the flags
 * leave the choice to the library and do not set KDA_FLAG_SPLIT_FULL_RERUN
 * (1 = one pass); 0 for invalid sizes.
 */
int kda_chunk_fwd_auto_segments(int64_t B, int64_t T, int64_t H,
                                int64_t dk, int64_t dv, int dtype);

/*
 * The plan kda_chunk_fwd (and kda_chunk_fwd_gated) follows for these sizes
 * and flags when its workspace holds what the library asks for:
 *   *segments  : segments per sequence (1 = one pass; a requested count is
 *                reported as the count its 32-token-aligned length gives)
 *   *per_chain : 1 when one workgroup covers a whole chain's 128 state
 *                columns, 0 when one covers a 64-column slice (and for every
 *                shape outside the pipelined path)
 *   *guarded   : 1 when the library's two-segment split is guarded: a probe
 *                launch first runs the second segment's transitions for a
 *                few chunks, and the split runs only if every chain's
 *                transition vanished there; otherwise the one pass (the plan
 *                with KDA_FLAG_SEGMENTS(1)) runs instead, decided on the
 *                device (no host synchronisation).  Picked where gates that
 *                keep memory would make the split slower than one pass.
 * The flags that matter: the segment bits, KDA_FLAG_SPLIT_FULL_RERUN,
 * KDA_FLAG_PAIRWISE_DIAGONAL and the workgroup layout flags.  Returns KDA_OK,
 * or the error the call would give for sizes or flags it rejects (outputs
 * untouched).  Host only: launches nothing.
 */
int kda_chunk_fwd_plan(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int dtype,
                       unsigned flags, int *segments, int *per_chain, int *guarded);

/*
 * As kda_chunk_fwd_workspace_size for an explicit segment count (the value
 * of the KDA_FLAG_SEGMENTS bits: 0 = the library's choice with or without
 * KDA_FLAG_SPLIT_FULL_RERUN, 1 = no split).  Returns 0 for invalid sizes or
 * a count above 255.
 */
size_t kda_chunk_fwd_workspace_size_segments(int64_t B, int64_t T, int64_t H,
                                             int64_t dk, int64_t dv, int dtype, int nseg);

/*
 * kda_chunk_fwd -- chunkwise prefill over T tokens for B x H independent
 * chains, 64-token chunks built from four 16-token subtiles.
 *   ("Kimi K3 internal structure analysis", section "Sequence mixing: 3 KDA
 *   layers per global MLA layer": the gate floor keeps each 16-token tile's
 *   cumulative log-decay inside (-80, 0), so the diagonal and the
 *   off-diagonal causal tiles are all dense matrix products.)
 *   q, k          : [B, T, H, dk] dtype
 *   v             : [B, T, H, dv] dtype
 *   g             : [B, T, H, dk] fp32, each value in [-5, 0] (e.g. from kda_gate)
 *   beta          : [B, T, H]     dtype
 *   initial_state : [B, H, dk, dv] fp32, or NULL for a zero state
 *   final_state   : [B, H, dk, dv] fp32, or NULL if not wanted; it may equal
 *                   initial_state (in-place continuation)
 *   o             : [B, T, H, dv] dtype (output; must not alias any input)
 *   workspace     : device buffer of at least kda_chunk_fwd_workspace_size()
 *                   bytes (..._size_segments() for an explicit segment count);
 *                   required with KDA_FLAG_CHECK_RANGE, explicit segments,
 *                   or fp32 inputs at dk = 128 (per-chunk buffers of the
 *                   fp32 16-token path, about 1.6 KB per token and chain).
 *                   May be NULL or smaller otherwise: the library then
 *                   picks among the segment counts whose buffers fit (one
 *                   pass when none does).
 * Chunks and 16-token tiles are aligned to token 0 of the call; the last
 * chunk may be partial.  Accumulation and the carried state are fp32.
 *
 * Sequence-parallel path ("Kimi K3 internal structure analysis", section
 * "Infrastructure for a 3T-class MoE": a sequence segment maps an incoming
 * state to an outgoing one).  When the chains alone do not fill the GPU
 * (bf16, dk = 128, dv in {64, 128}), each sequence is cut into P segments of
 * equal 32-token-aligned length; the count and the workgroup layout (one
 * workgroup per chain or per 64-column slice, see
 * KDA_FLAG_WORKGROUP_PER_CHAIN) minimise a model of the wall time: rounds of
 * workgroups per launch times the segment length, plus the chaining steps,
 * with the transitions priced as vanishing 2% of the way into a segment
 * (kda_chunk_fwd_plan reports the choice).  The recurrence is affine in the
 * state, S_end = M S_start + L, so three stream-ordered launches give the
 * same result as one pass up to fp32 rounding:
 *   1. segment 0 from initial_state (its o is final); every other segment
 *      from a zero state (L, and its o) and its transition M (v = 0,
 *      identity start), noting the chunk after which M is exactly zero;
 *   2. the segments' initial states, chained as M S + L;
 *   3. segments 1 .. P-1 again from their initial states, writing o and
 *      (last segment) final_state, up to that chunk only: from there on
 *      the incoming state's image M S is zero (the decay of every channel
 *      has underflowed fp32), so the zero-start o of step 1 stands and the
 *      last segment's final state is its L.
 * How far step 3 runs depends on the gates: a chunk or two when every
 * channel decays fast, the whole segment when some channel keeps memory
 * past its end (KDA_FLAG_SPLIT_FULL_RERUN then picks a count for that case
 * and leaves the last segment out of step 1).  The outputs computed in
 * step 3 and those kept from step 1 each agree with one pass to fp32
 * rounding.  The library picks P; KDA_FLAG_SEGMENTS(n) forces it (tests).
 * Where the library's choice is two segments and one pass would be faster
 * if no transition vanished (chains enough to fill the GPU in one pass of
 * 64-column slices), the split is guarded: a first launch runs each chain's
 * second-segment transition for a few chunks (2% of the segment, at least
 * eight) and records where it vanished; the split's launches run only if
 * every chain's did, else a one-pass launch runs; each launch reads the
 * records and returns at once when it is not the path taken, so the choice
 * needs no host synchronisation.  The result is then bit-identical to the
 * forced split or to the forced one pass.  The split uses the workspace; the
 * automatic choice takes the best count whose buffers fit in it (one pass
 * when none does).  Non-finite inputs stay in their chain in
 * every path; inside it, one pass carries a NaN or Inf in the state to the
 * end, while the stopping split applies a transition found exactly zero as
 * zero (it takes L for M S + L and keeps the zero-start outputs), so the
 * non-finite value does not pass such a point.
 */
int kda_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                  const void *beta, const float *initial_state, float *final_state,
                  void *o, void *workspace, size_t workspace_bytes,
                  int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                  int dtype, unsigned flags, void *stream);

/*
 * kda_chunk_fwd_gated -- kda_gate and kda_chunk_fwd as one call: the gate
 * g = -5 sigmoid(exp(A) z) of the same section of "Kimi K3 internal structure
 * analysis" is evaluated where the chunk kernel loads each chunk, so g never
 * goes through device memory.
 *   z : [B, T, H, dk] dtype (input, as given to kda_gate)
 *   A : [H, dk]       fp32  (input)
 * Every other argument is as for kda_chunk_fwd (g is not taken).  The gate is
 * evaluated with the hardware base-2 exponential and reciprocal: alpha agrees
 * with exp(kda_gate's g) to a few fp32 ulp, so o and final_state agree with
 * kda_gate followed by kda_chunk_fwd to fp32 rounding, not bit for bit.
 * bf16 inputs with dk = 128 and dv in {64, 128} run fused (the workspace is
 * then exactly what kda_chunk_fwd takes, including the sequence split and
 * KDA_FLAG_PAIRWISE_DIAGONAL); other shapes run the gate kernel into the
 * start of the workspace first.  KDA_FLAG_CHECK_RANGE is rejected
 * (INVALID_ARGUMENT): the gate's floor bounds g by construction.
 */
size_t kda_chunk_fwd_gated_workspace_size(int64_t B, int64_t T, int64_t H,
                                          int64_t dk, int64_t dv, int dtype);
int kda_chunk_fwd_gated(const void *q, const void *k, const void *v, const void *z,
                        const float *A, const void *beta, const float *initial_state,
                        float *final_state, void *o, void *workspace, size_t workspace_bytes,
                        int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                        int dtype, unsigned flags, void *stream);

/*
 * kda_chunk_fwd_gated_noalloc -- kda_chunk_fwd_gated for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The same arguments without the workspace;
 * the call's scratch is a fixed device array inside the library,
 * KDA_NOALLOC_SCRATCH_BYTES (32 MiB) on each GPU it runs on, held from the
 * first call on that GPU until the process ends.
 *  - What the scratch holds: the sequence split's per-segment states and
 *    transitions (bf16, dk = 128, dv in {64, 128}), or the staged g
 *    (B*T*H*dk*4 bytes) of shapes without the fused gate.
 *  - Sizes: the automatic segment count is the best whose buffers fit in the
 *    array (one pass when none does, as kda_chunk_fwd_gated chooses within a
 *    smaller workspace).  An explicit KDA_FLAG_SEGMENTS(n), or a staged g, that
 *    needs more than the array returns KDA_ERR_INVALID_ARGUMENT before any
 *    launch; kda_last_error() gives the bytes needed.
 *  - No call allocates or frees device memory, and no part of the array has
 *    to start at zero: every word a call reads was written earlier in that
 *    call.
 *  - Every call on one GPU shares that GPU's array, which keeps the last
 *    call's contents: calls that overlap in time on one GPU (other streams or
 *    host threads without ordering between them) race and give wrong results.
 *    Order them on one stream.
 *  - The first call on a GPU looks up the array's address there (on the
 *    device `stream` belongs to); KDA_ERR_HIP if that fails.
 *  - Under HIP graph capture: make one call on that GPU before capturing (the
 *    address lookup), and leave out KDA_FLAG_CHECK_RANGE, which clears a
 *    counter, reads it back to the host and waits for it.  Without it a call
 *    issues kernel launches only.
 * With the same segment count the results equal kda_chunk_fwd_gated's bit
 * for bit (the same kernels run).
 */
#define KDA_NOALLOC_SCRATCH_BYTES (32u << 20)
int kda_chunk_fwd_gated_noalloc(const void *q, const void *k, const void *v, const void *z,
                                const float *A, const void *beta, const float *initial_state,
                                float *final_state, void *o, int64_t B, int64_t T, int64_t H,
                                int64_t dk, int64_t dv, int dtype, unsigned flags, void *stream);

/*
 * kda_decode_step -- one token for each of N independent sequences x H heads,
 * with the gate fused and the state updated IN PLACE (read once, written once).
 *   (The studioglobal.ai summary of the Kimi K3 report, KDA section: a
 *   fixed-size recurrent state, so the work per decoded token does not grow
 *   with the context.)
 *   q, k, z : [N, H, dk] dtype
 *   v       : [N, H, dv] dtype
 *   beta    : [N, H]     dtype
 *   A       : [H, dk]    fp32
 *   state   : [N, H, dk, dv] fp32, read and overwritten with the new state
 *   o       : [N, H, dv] dtype (output; must not alias any input)
 */
int kda_decode_step(const void *q, const void *k, const void *v, const void *z,
                    const float *A, const void *beta, float *state, void *o,
                    int64_t N, int64_t H, int64_t dk, int64_t dv,
                    int dtype, void *stream);

/*
 * kda_chunk_bwd -- gradients of L = <o, d_o> + <S_T, d_final_state> through
 * the recurrence kda_chunk_fwd computes (same inputs and layouts), with
 * respect to q, k, v, g, beta and the initial state.  The step it reverses
 * is the one of "Kimi K3 internal structure analysis", section "Sequence
 * mixing: 3 KDA layers per global MLA layer" (retention, delta-rule write,
 * read after the write); the pages say nothing of training, so the reverse
 * mode is derived from that step.
 * Default path: 16-token chunks with fp32 matrix-core products -- the state
 * entering every even chunk (forward pass) and the gradient leaving every
 * odd one (reverse pass) go to the workspace, then the token gradients of
 * all chunk pairs are formed at once.  It relies on the range the gate floor guarantees (every 16-token
 * sum of g from the sequence start >= -80; KDA_FLAG_CHECK_RANGE verifies it
 * as kda_chunk_fwd does).  KDA_FLAG_TOKEN_BACKWARD selects the token-level
 * reverse mode (state checkpoints every 8 tokens), which takes any g <= 0.
 *   d_o             : [B, T, H, dv] dtype
 *   d_final_state   : [B, H, dk, dv] fp32, or NULL (zero)
 *   dq, dk, dg      : [B, T, H, dk] fp32 (outputs)
 *   dv              : [B, T, H, dv] fp32 (output)
 *   dbeta           : [B, T, H]     fp32 (output)
 *   d_initial_state : [B, H, dk, dv] fp32, or NULL if not wanted
 *   workspace       : see the sizes below
 *   flags           : KDA_FLAG_CHECK_RANGE (chunked path only), KDA_FLAG_TOKEN_BACKWARD
 * Outputs must not alias inputs.  KDA_ERR_RANGE as for kda_chunk_fwd.
 *
 * Workspace.  Both paths keep per-token buffers, so a whole-sequence
 * workspace grows linearly with T: about 6.8 KiB per token and chain for the
 * chunked path at dk = dv = 128 (the states entering even 16-token chunks and
 * the gradients leaving odd ones, X/P/At, W, dU and the decayed operands), and
 * 8 KiB plus per-slice partial gradients for the token path (a state every 8
 * tokens).  The chunked path therefore also runs in segments: given less than
 * the whole-sequence size, it takes the longest segment (a multiple of 32
 * tokens) whose buffers fit, sweeps the forward state pass over the segments
 * to get the state entering each, then runs the segments in reverse, carrying
 * the state gradient back (the forward state pass runs twice).  Its
 * workspace is then bounded by one segment plus (segments + 1) B H dk dv fp32
 * states, e.g. B1 H32 T1M d128 in 32768-token segments takes about 7.2 GB
 * instead of about 230 GB.  The token path needs its whole-sequence size.
 *   kda_chunk_bwd_workspace_size        : the whole-sequence size of the
 *                                         larger path (fits every call)
 *   kda_chunk_bwd_workspace_size_flags  : the size for the path `flags`
 *                                         selects; segment_tokens = 0 for the
 *                                         whole sequence in one segment, n > 0
 *                                         for segments of n tokens (rounded up
 *                                         to 32; chunked path only), or
 *                                         KDA_BWD_SEGMENTS_MIN_WORKSPACE for the
 *                                         smallest over all segment lengths:
 *                                         the least kda_chunk_bwd accepts
 *                                         (INVALID_ARGUMENT below it).
 */
#define KDA_BWD_SEGMENTS_MIN_WORKSPACE ((int64_t)-1)
size_t kda_chunk_bwd_workspace_size(int64_t B, int64_t T, int64_t H,
                                    int64_t dk, int64_t dv, int dtype);
size_t kda_chunk_bwd_workspace_size_flags(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                          int dtype, unsigned flags, int64_t segment_tokens);
int kda_chunk_bwd(const void *q, const void *k, const void *v, const float *g,
                  const void *beta, const float *initial_state, const void *d_o,
                  const float *d_final_state, float *dq, float *dk, float *dv, float *dg,
                  float *dbeta, float *d_initial_state, void *workspace, size_t workspace_bytes,
                  int64_t B, int64_t T, int64_t H, int64_t dk_dim, int64_t dv_dim,
                  int dtype, unsigned flags, void *stream);

/*
 * State pool for serving ("Kimi K3 internal structure analysis", section
 * "Serving two incompatible cache types": the KDA layers keep a fixed-size
 * recurrent state per sequence beside the MLA layers' growing cache).  A pool
 * holds n_slots states, [n_slots, H, dk, dv] fp32; each call names the slot
 * of each of its sequences in an int32 device array `slots` (4-byte aligned).
 * The pooled calls compute exactly what their plain counterparts compute on
 * the states gathered from those slots, and write the new states back to the
 * same slots in place.  A slot outside [0, n_slots) skips its sequence: none
 * of its state or output is read or written.  Two sequences of one call must
 * not share a slot (their writes would race); the library does not check.
 */

/* Zero the states of the n slots listed in `slots` (a sequence starting). */
int kda_state_pool_reset(float *state_pool, const int32_t *slots, int64_t n,
                         int64_t n_slots, int64_t H, int64_t dk, int64_t dv,
                         void *stream);

/*
 * kda_chunk_fwd with each sequence's initial and final state in the pool:
 * sequence b (of B, all T tokens long) starts from slot slots[b] and leaves
 * its final state there.  q, k, v, g, beta, o, workspace, flags as in
 * kda_chunk_fwd (the sequence split applies as well).
 */
int kda_chunk_fwd_pooled(const void *q, const void *k, const void *v, const float *g,
                         const void *beta, float *state_pool, const int32_t *slots,
                         void *o, void *workspace, size_t workspace_bytes,
                         int64_t B, int64_t T, int64_t n_slots, int64_t H,
                         int64_t dk, int64_t dv, int dtype, unsigned flags, void *stream);

/*
 * kda_chunk_fwd_pooled for B sequences of different lengths packed along the
 * token axis: q, k [total_tokens, H, dk], v, o [total_tokens, H, dv], g
 * [total_tokens, H, dk] fp32, beta [total_tokens, H]; sequence b is rows
 * cu_seqlens[b] .. cu_seqlens[b+1]-1 (cu_seqlens: B+1 int64 on the device,
 * non-decreasing from 0; values outside [0, total_tokens] are clamped there,
 * so a bad table cannot address outside the tensors).  An empty sequence
 * leaves its slot unchanged.  bf16, dk = 128, dv in {64, 128}; one pass (no
 * sequence split, no range check); the position-pair flag applies.
 */
int kda_chunk_fwd_varlen_pooled(const void *q, const void *k, const void *v, const float *g,
                                const void *beta, float *state_pool, const int32_t *slots,
                                const int64_t *cu_seqlens, void *o, int64_t B,
                                int64_t total_tokens, int64_t n_slots, int64_t H, int64_t dk,
                                int64_t dv, int dtype, unsigned flags, void *stream);

/*
 * kda_chunk_fwd_varlen_pooled with the gate evaluated inside the chunk kernel
 * (as kda_chunk_fwd_gated): z [total_tokens, H, dk] in the input dtype and A
 * [H, dk] fp32 instead of g.  Same shapes, layout and rules otherwise
 * (KDA_FLAG_CHECK_RANGE is rejected, as everywhere the gate is fused).
 */
int kda_chunk_fwd_varlen_pooled_gated(const void *q, const void *k, const void *v, const void *z,
                                      const float *A, const void *beta, float *state_pool,
                                      const int32_t *slots, const int64_t *cu_seqlens, void *o,
                                      int64_t B, int64_t total_tokens, int64_t n_slots, int64_t H,
                                      int64_t dk, int64_t dv, int dtype, unsigned flags,
                                      void *stream);

/*
 * kda_decode_step for N sequences whose states live in the pool: sequence n
 * reads and updates slot slots[n] in place (continuous batching: the set of
 * slots may change from step to step).  q, k, v, z, A, beta, o as in
 * kda_decode_step.
 */
int kda_decode_step_pooled(const void *q, const void *k, const void *v, const void *z,
                           const float *A, const void *beta, float *state_pool,
                           const int32_t *slots, void *o, int64_t N, int64_t n_slots,
                           int64_t H, int64_t dk, int64_t dv, int dtype, void *stream);

/* Message describing the last failed call on this thread ("" if none). */
const char *kda_last_error(void);

/* Library version string. */
const char *kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
