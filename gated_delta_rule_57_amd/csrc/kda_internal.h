// Internal interface between the C-ABI host code and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// One launch of the fused chunk kernel.  The sequence of each (b, h) is cut
// into nseg segments of seg_len tokens (the last one may be shorter); every
// (b, segment, h) is walked by its own workgroups.
//   mode 0 (outputs): segment j starts from initial state s0 when nseg == 1,
//     else from seg_in[b, j, h]; o and checkpoints are written, and the last
//     segment writes s_final.
//   mode 1 (segment summaries, segments 0..nseg-2): "Z" workgroups run the
//     segment from a zero state (segment 0 from s0) and store the state at its
//     end in seg_z[b, j, h] (dk x dv); "P" workgroups (segments >= 1) run it
//     with v = 0 from the identity and store the segment's transition matrix in
//     seg_p[b, j, h] (dk x dk).  Nothing else is written.
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* beta;
  const float* s0;
  void* o;
  float* s_final;
  float* ck;
  int64_t B, T, H, ck_every;
  int64_t seg_len, nseg;
  int mode;
  const float* seg_in;
  float* seg_z;
  float* seg_p;
  // checkpoints at listed positions instead of every ck_every tokens: ck_pos
  // (device, n_ck entries) holds token counts; entry i of ck is the state after
  // ck_pos[i] tokens, written only if that is a chunk end in (0, T]
  const int64_t* ck_pos;
  int64_t n_ck;
  // g holds raw decay logits a (log-decay = -softplus(a)) instead of log-decays
  int gate_logits;
  // output gate z [B, T, H, dv] (input dtype) or NULL: o = (S^T q) * sigmoid(z)
  const void* ogate;
  // range-check flag word (device) of a build with KDA_DEBUG_RANGE, else NULL
  unsigned* range_flags;
  // When seg_count > 0 the launch covers segments seg_first .. seg_first + seg_count - 1
  // only (instead of the ranges above), and a mode-1 launch has transition ("P")
  // workgroups only if with_p.  Used by the split summary pass (chunk_fwd_summary).
  int64_t seg_first = 0, seg_count = 0;
  int with_p = 1;
};

// d_v slice width per prefill workgroup.
int prefill_slice(int dk, int dv, bool in_bf16);

// Number of workgroups of one prefill launch over `units` (b, segment, h)
// triples with `slices` workgroups each.
int64_t prefill_grid(int64_t units, int slices);

hipError_t chunk_fwd(const PrefillArgs& a, int dk, int dv, bool in_bf16, bool out_bf16,
                     hipStream_t s);

// Whether the split summary pass below serves these sizes (bfloat16 inputs, d_k = d_v =
// 128, 64-token chunks).
bool summary_split_ok(int dk, int dv, bool in_bf16, int chunk);

// The summary pass (mode 1) of a segmented launch as one kernel of two parts: the
// workgroups of segment 0 (a0: from the initial state, writing that segment's outputs,
// no transition workgroups) and, for segments 1 .. nseg-2 (a1), one workgroup for the
// zero-start state and one for the transition, each carrying all 128 columns and none
// of the query or output work.
hipError_t chunk_fwd_summary(const PrefillArgs& a0, const PrefillArgs& a1, bool out_bf16,
                             hipStream_t s);

// The pipelined kernel for 32- or 16-token chunks (bfloat16 inputs; slices of 64 value
// columns); same arguments and modes as chunk_fwd.
hipError_t chunk_fwd_pipe(const PrefillArgs& a, int chunk, int dk, int dv, bool out_bf16,
                          hipStream_t s);

// Entry states of the segments after the first: seg_in[b, 1, h] = seg_z[b, 0, h] (the
// summary of segment 0 starts from the initial state), seg_in[b, j+1, h] =
// seg_p[b, j, h] seg_in[b, j, h] + seg_z[b, j, h].  Slot 0 is not written.  float32.
hipError_t segment_scan(const float* seg_z, const float* seg_p, float* seg_in,
                        int64_t B, int64_t H, int64_t nseg, int dk, int dv, hipStream_t s);

// K draft tokens per sequence ([N, K, H, .] inputs): commit = false writes o for
// every token and leaves the state; commit = true advances the state in place by
// accept[n] tokens (clamped to [0, K]) and writes no o.
hipError_t multi_token(const void* q, const void* k, const void* v, const void* g,
                       const void* beta, const int32_t* accept, float* state, void* o, int64_t N,
                       int64_t K, int64_t H, int dk, int dv, bool in_bf16, bool out_bf16,
                       bool commit, hipStream_t s);

// ogate: output gate z [nh, dv] (input dtype) or NULL; o = (S^T q) * sigmoid(z)
hipError_t decode_step(const void* q, const void* k, const void* v, const void* g,
                       const void* beta, float* state, void* o, int64_t nh, int dk, int dv,
                       bool in_bf16, bool out_bf16, hipStream_t s, bool gate_logits = false,
                       const void* ogate = nullptr);

}  // namespace kda
