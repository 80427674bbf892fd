/*
 * kda.h - C ABI of the Kimi Delta Attention (KDA) library for AMD MI355X (gfx950).
 *
 * KDA is the fixed-size-state sequence mixer of the Kimi K3 hybrid model.  Per
 * batch row b and head h it carries a d_k x d_v state S and, for every token t,
 *
 *     g'_t = min(max(g_t, -5), 0)                       (per key channel)
 *     S_t  = (I - beta_t k_t k_t^T) Diag(exp g'_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t  = S_t^T q_t
 *
 * Sources (the pages' formulas were lost in extraction; the form above is the
 * standard one for the lineage they describe):
 *   - the delta rule -> scalar forget gate -> per-channel ("diagonal") gate
 *     lineage, and the negative-softplus decay logits: Towards-AI article on the
 *     Kimi K3 report, section "Kimi Delta Attention (KDA)";
 *   - the -5 floor on the log-decay (each step keeps at least ~0.67% of a
 *     channel) and its consequence that a 16-token tile's cumulative log-decay
 *     stays in [-80, 0], so diagonal tiles of the chunked form run as the same
 *     dense matrix product as off-diagonal tiles: orkas.ai blog "Kimi K3
 *     architecture", section "A lower bound that deleted a GPU code path";
 *   - the in-place recurrent state update of decoding: same blog, section
 *     "The cost is paid in the serving stack".
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers (HBM of the current HIP device),
 *     row-major and contiguous.  Token tensors are [B, T, H, D]; states are
 *     [B, H, d_k, d_v] float32 (rows = key channels).
 *   - The caller owns every buffer.  The library never allocates device
 *     memory, keeps no global mutable state, and never synchronises: work is
 *     enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     execution errors surface at the caller's next synchronisation.
 *   - Arguments are validated on the host before anything is launched; a
 *     non-OK status means nothing was enqueued.  KDA_ERR_HIP reports a failed
 *     launch (hipGetLastError after the enqueue).
 *   - Supported sizes: d_k, d_v in {64, 128}; T >= 1; chunk 64, or 32 and 16
 *     with bfloat16 inputs.  float32 inputs support d_k = d_v = 64 (the
 *     float32-parity configuration); bfloat16 inputs support all four (d_k, d_v)
 *     pairs.  The chunked kernels address a chunk's token rows by 32-bit byte
 *     offsets, so H may be at most (2^32 - 1) / (256 max(d_k, d_v)) (131,071 at
 *     d = 128); larger H is KDA_ERR_SHAPE.
 *   - Pointers must be 16-byte aligned.
 *   - Concurrent calls on different streams are safe (the library is
 *     stateless); calls that write the same buffers race.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Size of the device scratch array that kda_chunk_fwd_noalloc uses as its
 * workspace (64 MiB per GPU). */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)

/* The two enumerations carry range sentinels (never valid arguments, never returned):
 * they make every int a value of the type, so that a bad value passed from C or
 * through a foreign-function interface is reported (KDA_ERR_DTYPE; "KDA_ERR_UNKNOWN")
 * instead of being an out-of-range enumeration value inside the C++ library. */
typedef enum {
  KDA_F32 = 0,
  KDA_BF16 = 1,
  KDA_DTYPE_RANGE_MIN_ = -0x7fffffff - 1,
  KDA_DTYPE_RANGE_MAX_ = 0x7fffffff
} kda_dtype_t;

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = -1,      /* a required pointer is NULL */
  KDA_ERR_SHAPE = -2,     /* unsupported or inconsistent sizes */
  KDA_ERR_DTYPE = -3,     /* unsupported dtype combination */
  KDA_ERR_ALIGN = -4,     /* a pointer is not 16-byte aligned */
  KDA_ERR_WORKSPACE = -5, /* workspace missing or too small */
  KDA_ERR_ALIAS = -6,     /* an output overlaps an input it may not overlap */
  KDA_ERR_HIP = -7,       /* the HIP runtime reported an error at launch */
  KDA_STATUS_RANGE_MIN_ = -0x7fffffff - 1,
  KDA_STATUS_RANGE_MAX_ = 0x7fffffff
} kda_status_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* kda_status_str(kda_status_t status);

/* Bytes of device workspace kda_chunk_fwd needs for these sizes (0 if none:
 * one segment, see kda_chunk_fwd_segment_tokens).  Returns 0 as well for
 * unsupported sizes; kda_chunk_fwd then reports why. */
size_t kda_chunk_fwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int dk, int dv, int chunk,
                                     kda_dtype_t in);

/*
 * kda_chunk_fwd - chunked parallel forward (prefill) over whole sequences.
 *
 * Computes o_t for t = 0..T-1 and the state after token T for every (b, h),
 * starting from `initial_state`, by the recurrence above, evaluated in chunks
 * of `chunk` tokens (the chunk-parallel rewrite the Towards-AI article's "Kimi
 * Delta Attention (KDA)" section names as the usual linear-attention layout).
 *
 *   q, k          [B, T, H, dk]  dtype `in`   query / key (not normalised here)
 *   v             [B, T, H, dv]  dtype `in`
 *   g             [B, T, H, dk]  dtype `in`   log-decay (clamped to [-5, 0]
 *                                             here; NaN propagates)
 *   beta          [B, T, H]      dtype `in`   write strength, used as given
 *   initial_state [B, H, dk, dv] float32      NULL = zeros
 *   o             [B, T, H, dv]  dtype `out`  written
 *   final_state   [B, H, dk, dv] float32      written; NULL = not wanted.
 *                                             May equal initial_state exactly
 *                                             (in-place update); any other
 *                                             overlap is KDA_ERR_ALIAS.
 *   checkpoints   [B, T / checkpoint_every, H, dk, dv] float32, or NULL.
 *                 Entry j is the state after token checkpoint_every*(j+1).
 *   checkpoint_every  0 = off; else a positive multiple of `chunk`.
 *   chunk         64, or (bfloat16 inputs) 32 or 16.  64 runs a fused kernel
 *                 whose phases take turns over one chunk; 32 and 16 run a
 *                 pipelined kernel in which producer waves build chunk n+1's
 *                 state-independent operands while consumer waves advance the
 *                 state through chunk n.  All three compute the same result to
 *                 within rounding.
 *   workspace / workspace_bytes  at least kda_chunk_fwd_workspace_bytes(...)
 *                 bytes (may be NULL when that is 0), else KDA_ERR_WORKSPACE.
 *                 Must not overlap any other buffer.
 *
 * When B * H heads are too few to occupy the GPU, the sequences are cut into
 * segments (kda_chunk_fwd_segment_tokens reports the length) and the call
 * proceeds as kda_chunk_fwd_segmented below; the workspace holds the segments'
 * summaries and entry states.
 *
 * T need not be a multiple of `chunk`: the tail is padded inside the kernel
 * with beta = 0, g = 0 tokens, which leave the state unchanged.
 */
kda_status_t kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g,
                           const void* beta, const float* initial_state, void* o,
                           float* final_state, float* checkpoints, int64_t checkpoint_every,
                           int64_t B, int64_t T, int64_t H, int dk, int dv, int chunk,
                           kda_dtype_t in, kda_dtype_t out, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * kda_chunk_fwd_segmented - kda_chunk_fwd with the sequence cut into segments.
 *
 * Same arguments, outputs and errors as kda_chunk_fwd, plus `segment_tokens`
 * (a positive multiple of `chunk`).  Each sequence is cut into
 * ceil(T / segment_tokens) segments; segment_tokens >= T is one segment, the
 * same computation as kda_chunk_fwd's single pass.  With several segments
 * three launches are enqueued:
 *   1. every segment but the last is summarised in parallel: Z, the state it
 *      reaches from a zero state, and P (dk x dk), the product of its tokens'
 *      transitions, obtained by running it from the identity with v = 0; the
 *      first segment instead runs from initial_state and also writes its o and
 *      checkpoints (it is then done);
 *   2. a prefix scan over segments, S_in(j+1) = P_j S_in(j) + Z_j, gives every
 *      later segment's entry state;
 *   3. every segment after the first is run from its entry state, writing o,
 *      checkpoints and (last segment) final_state.
 * The segment law is the one the orkas.ai blog "Kimi K3 architecture" states
 * for splitting a sequence across devices (section "The cost is paid in the
 * serving stack"); here it spreads few long sequences over the GPU's compute
 * units.  The results agree with the one-segment path to within rounding (not
 * bitwise: the summaries take a different order of operations).
 *
 *   workspace / workspace_bytes  at least
 *                 kda_chunk_fwd_segmented_workspace_bytes(...) bytes (NULL
 *                 allowed when that is 0); must not overlap any other buffer.
 */
kda_status_t kda_chunk_fwd_segmented(const void* q, const void* k, const void* v, const void* g,
                                     const void* beta, const float* initial_state, void* o,
                                     float* final_state, float* checkpoints,
                                     int64_t checkpoint_every, int64_t B, int64_t T, int64_t H,
                                     int dk, int dv, int chunk, kda_dtype_t in, kda_dtype_t out,
                                     int64_t segment_tokens, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Workspace bytes of kda_chunk_fwd_segmented for these sizes: 4 * B * nseg * H
 * * dk * (2 dv + dk) rounded up, 0 for one segment or unsupported sizes. */
size_t kda_chunk_fwd_segmented_workspace_bytes(int64_t B, int64_t T, int64_t H, int dk, int dv,
                                               int chunk, kda_dtype_t in,
                                               int64_t segment_tokens);

/* The segment length kda_chunk_fwd uses for these sizes (a multiple of 64; a
 * value >= T means one segment), or 0 for unsupported sizes.  Several segments
 * are chosen only when B * H is too small to occupy the GPU's compute units. */
int64_t kda_chunk_fwd_segment_tokens(int64_t B, int64_t T, int64_t H, int dk, int dv, int chunk,
                                     kda_dtype_t in);

/*
 * kda_recurrent_step - one decode step for N independent sequences.
 *
 * For every (n, h): S <- Diag(exp g') S; S <- S + beta k (v - S^T k)^T;
 * o = S^T q.  The state is updated IN PLACE (no copy is kept, so a step
 * cannot be undone; the orkas.ai blog's "The cost is paid in the serving
 * stack" section describes this property of KDA decoding).
 *
 *   q, k, g  [N, H, dk]      dtype `in`
 *   v        [N, H, dv]      dtype `in`
 *   beta     [N, H]          dtype `in`
 *   state    [N, H, dk, dv]  float32, read and overwritten
 *   o        [N, H, dv]      dtype `out`, must not overlap `state`
 */
kda_status_t kda_recurrent_step(const void* q, const void* k, const void* v, const void* g,
                                const void* beta, float* state, void* o, int64_t N, int64_t H,
                                int dk, int dv, kda_dtype_t in, kda_dtype_t out, void* stream);

/*
 * Raw decay logits.  These variants take, in place of g, the decay logits `a`
 * (same shape and dtype) and use g = -softplus(a) = -log(1 + e^a) before the
 * floor: the negative-softplus map of the Towards-AI article on the Kimi K3
 * report (section "Kimi Delta Attention (KDA)"), fused into the kernels' gate
 * preparation.  Everything else is as in kda_chunk_fwd / kda_recurrent_step.
 * In float32, log-decays above about -6e-8 (a < -16.6) round to 0.
 */
kda_status_t kda_chunk_fwd_gate_logits(const void* q, const void* k, const void* v, const void* a,
                                       const void* beta, const float* initial_state, void* o,
                                       float* final_state, float* checkpoints,
                                       int64_t checkpoint_every, int64_t B, int64_t T, int64_t H,
                                       int dk, int dv, int chunk, kda_dtype_t in, kda_dtype_t out,
                                       void* workspace, size_t workspace_bytes, void* stream);
kda_status_t kda_recurrent_step_gate_logits(const void* q, const void* k, const void* v,
                                            const void* a, const void* beta, float* state, void* o,
                                            int64_t N, int64_t H, int dk, int dv, kda_dtype_t in,
                                            kda_dtype_t out, void* stream);

/*
 * Fused output gate.  These variants take one more input, the gate projection
 *   gate  [B, T, H, dv] (prefill) or [N, H, dv] (decode), dtype `in`,
 * and write o_t = (S_t^T q_t) * sigmoid(gate_t) elementwise, sigmoid(z) = 1 / (1 + e^-z),
 * instead of S_t^T q_t: one gate value per token, head and value channel, projected
 * from the token's input by the caller, so each token chooses which channels of the
 * mixer's output pass.  The Towards-AI article on the Kimi K3 report gives K3's Gated
 * MLA layers such a gate and says KDA has a counterpart (section "Gated MLA and No
 * Position Encoding (NoPE)"); the logistic form is the plain reading where the page
 * names no function.  The gate is applied before the output is rounded to `out` (one
 * rounding).  States, checkpoints and everything else are as in kda_chunk_fwd /
 * kda_recurrent_step; `gate` must be 16-byte aligned, non-NULL (KDA_ERR_NULL) and must
 * not overlap o, the states or the workspace (KDA_ERR_ALIAS).  The projection that
 * produces `gate` (weights) stays with the caller.
 */
kda_status_t kda_chunk_fwd_output_gate(const void* q, const void* k, const void* v, const void* g,
                                       const void* beta, const void* gate,
                                       const float* initial_state, void* o, float* final_state,
                                       float* checkpoints, int64_t checkpoint_every, int64_t B,
                                       int64_t T, int64_t H, int dk, int dv, int chunk,
                                       kda_dtype_t in, kda_dtype_t out, void* workspace,
                                       size_t workspace_bytes, void* stream);
kda_status_t kda_recurrent_step_output_gate(const void* q, const void* k, const void* v,
                                            const void* g, const void* beta, const void* gate,
                                            float* state, void* o, int64_t N, int64_t H, int dk,
                                            int dv, kda_dtype_t in, kda_dtype_t out, void* stream);

/*
 * kda_chunk_fwd_checkpoints_at - kda_chunk_fwd with states saved at listed positions.
 *
 * Same as kda_chunk_fwd (same workspace) with checkpoint_every = 0, except that
 * checkpoint i is the state after `positions[i]` tokens:
 *   positions    [n_positions] int64, DEVICE memory, strictly increasing, each a
 *                multiple of `chunk` in (0, T].  An entry that is not such a
 *                position leaves its checkpoint untouched (the kernel never
 *                writes outside the checkpoint array).  8-byte aligned.
 *   checkpoints  [B, n_positions, H, dk, dv] float32.
 * This serves prefix caching that hashes fixed token blocks and keeps the
 * recurrent state only at a sparse subset of block ends (the orkas.ai blog "Kimi
 * K3 architecture", section "The cost is paid in the serving stack"); a cache hit
 * restores a checkpoint as `initial_state` of the following call.
 */
kda_status_t kda_chunk_fwd_checkpoints_at(const void* q, const void* k, const void* v,
                                          const void* g, const void* beta,
                                          const float* initial_state, void* o, float* final_state,
                                          float* checkpoints, const int64_t* positions,
                                          int64_t n_positions, int64_t B, int64_t T, int64_t H,
                                          int dk, int dv, int chunk, kda_dtype_t in,
                                          kda_dtype_t out, void* workspace, size_t workspace_bytes,
                                          void* stream);

/*
 * Speculative decoding without rollback.  A draft of K tokens per sequence is
 * checked against the committed state, and only the accepted prefix is
 * committed.  The state cannot be rolled back once updated in place, so what is
 * kept for a draft is its tokens' projected inputs (far smaller than the
 * state); the accepted prefix is replayed from them on chip.  This is the scheme
 * the orkas.ai blog "Kimi K3 architecture" names for speculative decoding
 * (section "The cost is paid in the serving stack").
 *
 * Draft tensors are [N, K, H, D] (token-major per sequence, like a prefill of
 * T = K): q, k, g [N, K, H, dk], v [N, K, H, dv], beta [N, K, H].
 */

/*
 * kda_recurrent_verify - outputs of K draft tokens from the committed state.
 *
 * o[n, j] = S_j^T q[n, j], with S_j the state after draft tokens 0..j applied to
 * `state` by the recurrence above; `state` [N, H, dk, dv] float32 is only read.
 *   o  [N, K, H, dv]  dtype `out`, must not overlap the inputs or the state.
 * Equal to K calls of kda_recurrent_step on a copy of the state.
 */
kda_status_t kda_recurrent_verify(const void* q, const void* k, const void* v, const void* g,
                                  const void* beta, const float* state, void* o, int64_t N,
                                  int64_t K, int64_t H, int dk, int dv, kda_dtype_t in,
                                  kda_dtype_t out, void* stream);

/*
 * kda_recurrent_commit - advance each sequence's state by its accepted prefix.
 *
 * For every (n, h) the first accept[n] draft tokens (clamped to [0, K]) are
 * applied to `state` IN PLACE; sequences with accept[n] <= 0 are untouched.
 *   accept  [N] int32, DEVICE memory (typically written by the verification step).
 *   k, g, v, beta as for kda_recurrent_verify (q is not needed; dtype `in`).
 * kda_recurrent_verify and then kda_recurrent_commit with accept[n] = K equals
 * K calls of kda_recurrent_step.
 */
kda_status_t kda_recurrent_commit(const void* k, const void* v, const void* g, const void* beta,
                                  const int32_t* accept, float* state, int64_t N, int64_t K,
                                  int64_t H, int dk, int dv, kda_dtype_t in, void* stream);

/*
 * kda_chunk_fwd_noalloc - kda_chunk_fwd for callers that cannot allocate.
 *
 * For callers that may not call hipMalloc or any allocating routine: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.  Same
 * computation, arguments, outputs and errors as kda_chunk_fwd, without the workspace
 * arguments: when the sizes call for the segment path, its workspace is a device
 * array inside the library, KDA_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, loaded with
 * the library and held until the process ends.  The call itself allocates nothing.
 *   - Sizes whose workspace (kda_chunk_fwd_workspace_bytes) exceeds
 *     KDA_NOALLOC_SCRATCH_BYTES return KDA_ERR_WORKSPACE before anything else is
 *     done; use kda_chunk_fwd with a workspace of your own for those.  (The
 *     segmentation the library picks keeps its workspace near 30 MiB at most for
 *     B <= 4, H <= 128, T <= 2^30, d = 128, so this is a guard.)
 *   - The first call on a device that needs the array looks up its address on that
 *     device (hipGetSymbolAddress; KDA_ERR_HIP if that fails); the address is kept
 *     per device.  Call with the device of `stream` current.
 *   - Every call on one GPU shares that GPU's array, and nothing in it needs to start
 *     at zero (each call writes what it reads).  Calls that overlap in time on one GPU
 *     (different streams, or threads) race on the array: serialise them.
 */
kda_status_t kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* g,
                                   const void* beta, const float* initial_state, void* o,
                                   float* final_state, float* checkpoints,
                                   int64_t checkpoint_every, int64_t B, int64_t T, int64_t H,
                                   int dk, int dv, int chunk, kda_dtype_t in, kda_dtype_t out,
                                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
