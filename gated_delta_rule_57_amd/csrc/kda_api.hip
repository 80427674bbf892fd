// Host side of the C ABI declared in include/kda.h: argument validation,
// dispatch to the gfx950 kernels, status codes.  Nothing here allocates device
// memory or synchronises.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <mutex>

#include "kda.h"
#include "kda_internal.h"
#ifdef KDA_DEBUG_RANGE
#include "kda_debug.h"
#endif

// Workspace of kda_chunk_fwd_noalloc: a file-scope device array, so that the call
// allocates nothing.  Every GPU the library runs on holds its own copy (loaded with
// the library's code object, kept until the process ends).  Host code never uses
// the array's name as an address: it uses the device address that
// hipGetSymbolAddress reports for the current device (scratch_address below).
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];


namespace {

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};

Span span(const void* p, int64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Span{a, a + (uintptr_t)bytes};
}

bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dtype_ok(kda_dtype_t d) { return d == KDA_F32 || d == KDA_BF16; }

int64_t esize(kda_dtype_t d) { return d == KDA_BF16 ? 2 : 4; }

bool head_dim_ok(int d) { return d == 64 || d == 128; }

// Guards against int64 overflow of element counts.
bool mul_ok(int64_t a, int64_t b) { return a >= 0 && b >= 0 && (b == 0 || a <= INT64_MAX / b); }

}  // namespace

extern "C" const char* kda_status_str(kda_status_t s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
    case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE: unsupported or inconsistent sizes";
    case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE: unsupported dtype";
    case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN: a pointer is not 16-byte aligned";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
    case KDA_ERR_ALIAS: return "KDA_ERR_ALIAS: an output overlaps an input";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: the HIP runtime reported an error";
    default: break;
  }
  return "KDA_ERR_UNKNOWN";
}

namespace {

constexpr int64_t kChunk = 64;
// Compute units of an MI355X.  The prefill kernel runs one workgroup per CU
// (its shared memory and register use admit no second one), so a launch of n
// workgroups takes ceil(n / kCUs) rounds.
constexpr int64_t kCUs = 256;

// The prefill kernel addresses one chunk's token rows as 32-bit byte offsets from the
// chunk's first row, row * H * d * element size (inputs, and the output in either
// dtype).  Sizes whose largest such offset does not fit 32 bits are rejected: H at most
// 131,071 for d = 128 (float32 output), far beyond any model's head count.
constexpr int64_t kMaxChunkSpanBytes = 0xffffffffLL;

// Chunk lengths: 64 (the default), 32 and 16 (bfloat16 inputs only).
bool chunk_ok(int chunk, kda_dtype_t in) {
  return chunk == 64 || ((chunk == 32 || chunk == 16) && in == KDA_BF16);
}

bool sizes_ok(int64_t B, int64_t T, int64_t H, int dk, int dv, int chunk, kda_dtype_t in) {
  if (!dtype_ok(in) || B < 1 || T < 1 || H < 1 || !head_dim_ok(dk) || !head_dim_ok(dv) ||
      !chunk_ok(chunk, in))
    return false;
  if (in == KDA_F32 && (dk != 64 || dv != 64)) return false;
  const int64_t dmax = dk > dv ? dk : dv;
  if (H > kMaxChunkSpanBytes / (kChunk * dmax * 4)) return false;
  // the byte spans of the token tensors (tokens x d x element size, at most 4 bytes)
  // stay inside int64
  return mul_ok(B, T) && mul_ok(B * T, H) && mul_ok(B * T * H, 4 * dmax);
}

int64_t num_segments(int64_t T, int64_t seg_len) { return seg_len >= T ? 1 : (T + seg_len - 1) / seg_len; }

// Segment length chosen by kda_chunk_fwd: the one that minimises a round count
// model of the three launches (summaries, scan, outputs) when that beats one
// segment by 20% or more; T rounded up to whole chunks (one segment) otherwise.
// Deterministic in the sizes.
int64_t auto_segment_tokens(int64_t B, int64_t T, int64_t H, int dk, int dv, bool bf16,
                            int chunk) {
  const int64_t nch = (T + kChunk - 1) / kChunk;
  const int sl = kda::prefill_slice(dk, dv, bf16);
  const int64_t ns = dv / sl, np = dk / sl;
  const bool split = kda::summary_split_ok(dk, dv, bf16, chunk);
  auto rounds = [](int64_t wgs) { return (double)((wgs + kCUs - 1) / kCUs); };
  const double one = rounds(B * H * ns) * (double)nch;
  double best = one;
  int64_t best_len = nch * kChunk;  // one segment
  for (int64_t want = 2; want <= 64 && want <= nch; ++want) {
    const int64_t segc = (nch + want - 1) / want;  // chunks per segment
    const int64_t n = (nch + segc - 1) / segc;     // segments that length gives
    if (n != want) continue;
    // summaries: zero-start states of segments 0 .. n-2 (segment 0 from the initial
    // state, writing its outputs too) and transitions of segments 1 .. n-2; outputs:
    // segments 1 .. n-1
    // (with the split summary pass, segments 1 .. n-2 take two 128-column workgroups
    // each, whose chunk steps cost about as much as an ordinary one)
    const int64_t wg_summary = (split && n >= 3) ? B * H * (ns + 2 * (n - 2))
                                                 : B * H * ((n - 1) * (ns + np) - np);
    const double summary = rounds(wg_summary) * (double)segc;
    const double outputs = rounds(B * (n - 1) * H * ns) * (double)segc;
    // a scan step costs about a third of a chunk step; the two extra launches
    // about a chunk step each
    const double extra = 0.3 * (double)n + 2.0;
    const double cost = summary + outputs + extra;
    if (cost < best) {
      best = cost;
      best_len = segc * kChunk;
    }
  }
  return best <= 0.8 * one ? best_len : nch * kChunk;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

#ifdef KDA_DEBUG_RANGE
// Range-check build: the chunk kernels OR violation bits into this device word (one
// copy per GPU), whose address is looked up once per device.
static __device__ unsigned range_flags_word;
constexpr int kMaxRangeDevices = 64;
std::mutex g_range_mu;
unsigned* g_range_ptr[kMaxRangeDevices];

hipError_t range_flags_address(unsigned** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxRangeDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_range_mu);
  if (!g_range_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(range_flags_word));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_range_ptr[dev] = static_cast<unsigned*>(p);
  }
  *out = g_range_ptr[dev];
  return hipSuccess;
}
#endif

// One launch of the chunk kernel for this chunk length: 64 tokens by the fused
// 64-token kernel, 32 and 16 by the pipelined one.
hipError_t launch_chunks(const kda::PrefillArgs& a, int chunk, int dk, int dv, bool in_bf16,
                         bool out_bf16, hipStream_t st) {
  if (chunk == 64) return kda::chunk_fwd(a, dk, dv, in_bf16, out_bf16, st);
  return kda::chunk_fwd_pipe(a, chunk, dk, dv, out_bf16, st);
}

// Workspace of the segmented path: entry states and end-from-zero states
// [B, nseg, H, dk, dv], transitions [B, nseg, H, dk, dk], float32.
size_t segment_workspace(int64_t B, int64_t H, int64_t nseg, int dk, int dv, size_t* off_z,
                         size_t* off_p) {
  if (nseg <= 1) return 0;
  const size_t n_in = align256((size_t)(B * nseg * H) * (size_t)dk * (size_t)dv * 4);
  const size_t n_p = align256((size_t)(B * nseg * H) * (size_t)dk * (size_t)dk * 4);
  if (off_z) *off_z = n_in;
  if (off_p) *off_p = 2 * n_in;
  return 2 * n_in + n_p;
}

kda_status_t chunk_fwd_impl(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const float* initial_state, void* o,
                            float* final_state, float* checkpoints, int64_t checkpoint_every,
                            int64_t B, int64_t T, int64_t H, int dk, int dv, int chunk,
                            kda_dtype_t in, kda_dtype_t out, int64_t seg_len, void* workspace,
                            size_t workspace_bytes, void* stream, const int64_t* ck_pos = nullptr,
                            int64_t n_ck = 0, bool gate_logits = false,
                            const void* ogate = nullptr, bool validate_only = false) {
  if (!q || !k || !v || !g || !beta || !o) return KDA_ERR_NULL;
  if ((checkpoint_every != 0 || n_ck != 0) && !checkpoints) return KDA_ERR_NULL;
  if (n_ck != 0 && !ck_pos) return KDA_ERR_NULL;
  if (n_ck < 0 || (n_ck > 0 && checkpoint_every != 0)) return KDA_ERR_SHAPE;
  if (ck_pos && (reinterpret_cast<uintptr_t>(ck_pos) & 7u) != 0) return KDA_ERR_ALIGN;
  if (!dtype_ok(in) || !dtype_ok(out)) return KDA_ERR_DTYPE;
  if (!sizes_ok(B, T, H, dk, dv, chunk, in)) return KDA_ERR_SHAPE;
  if (checkpoint_every < 0 || (checkpoint_every % chunk) != 0) return KDA_ERR_SHAPE;
  if (seg_len < 1 || seg_len % chunk != 0) return KDA_ERR_SHAPE;
  const int64_t nseg = num_segments(T, seg_len);
  const bool bf16 = in == KDA_BF16;
  const int sl = kda::prefill_slice(dk, dv, bf16);
  if (!mul_ok(B * H, nseg) || kda::prefill_grid(B * H * nseg, (dv + dk) / sl) > INT32_MAX)
    return KDA_ERR_SHAPE;
  size_t off_z = 0, off_p = 0;
  const size_t ws_need = segment_workspace(B, H, nseg, dk, dv, &off_z, &off_p);
  // validate_only: every check but the workspace's, then KDA_ERR_WORKSPACE when one is
  // needed (KDA_OK when none is); nothing is launched
  const bool ws_missing = ws_need > 0 && (!workspace || workspace_bytes < ws_need);
  if (ws_missing && !validate_only) return KDA_ERR_WORKSPACE;

  const void* ptrs[] = {q,           k,           v,         g,     beta, initial_state, o,
                        final_state, checkpoints, workspace, ogate};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KDA_ERR_ALIGN;

  const int64_t es = esize(in);
  const int64_t ntok = B * T * H;
  const int64_t heads = B * H;
  const Span sq = span(q, ntok * dk * es), sk = span(k, ntok * dk * es);
  const Span sv = span(v, ntok * dv * es), sg = span(g, ntok * dk * es);
  const Span sb = span(beta, ntok * es);
  // the output gate, if any, is one more input (an empty span otherwise)
  const Span sz = ogate ? span(ogate, ntok * dv * es) : Span{0, 0};
  const Span so = span(o, ntok * dv * esize(out));
  const int64_t state_bytes = heads * dk * dv * 4;
  const Span inputs[] = {sq, sk, sv, sg, sb, sz};
  for (const Span& s : inputs)
    if (overlaps(so, s)) return KDA_ERR_ALIAS;
  if (initial_state && overlaps(so, span(initial_state, state_bytes))) return KDA_ERR_ALIAS;
  if (final_state) {
    const Span sf = span(final_state, state_bytes);
    if (overlaps(sf, so)) return KDA_ERR_ALIAS;
    for (const Span& s : inputs)
      if (overlaps(sf, s)) return KDA_ERR_ALIAS;
    if (initial_state && initial_state != final_state &&
        overlaps(sf, span(initial_state, state_bytes)))
      return KDA_ERR_ALIAS;
  }
  const int64_t nck = n_ck > 0 ? n_ck : (checkpoint_every ? T / checkpoint_every : 0);
  if (!mul_ok(B * H, nck) || !mul_ok(B * H * nck, (int64_t)dk * dv * 4)) return KDA_ERR_SHAPE;
  if (checkpoints && nck > 0) {
    const Span sc = span(checkpoints, B * nck * H * dk * dv * 4);
    if (overlaps(sc, so)) return KDA_ERR_ALIAS;
    for (const Span& s : inputs)
      if (overlaps(sc, s)) return KDA_ERR_ALIAS;
    if (initial_state && overlaps(sc, span(initial_state, state_bytes))) return KDA_ERR_ALIAS;
    if (final_state && overlaps(sc, span(final_state, state_bytes))) return KDA_ERR_ALIAS;
  }
  if (ws_need > 0 && !ws_missing) {
    const Span sw = span(workspace, (int64_t)ws_need);
    for (const Span& s : inputs)
      if (overlaps(sw, s)) return KDA_ERR_ALIAS;
    if (overlaps(sw, so)) return KDA_ERR_ALIAS;
    if (initial_state && overlaps(sw, span(initial_state, state_bytes))) return KDA_ERR_ALIAS;
    if (final_state && overlaps(sw, span(final_state, state_bytes))) return KDA_ERR_ALIAS;
    if (checkpoints && nck > 0 && overlaps(sw, span(checkpoints, B * nck * H * dk * dv * 4)))
      return KDA_ERR_ALIAS;
  }

  if (validate_only) return ws_missing ? KDA_ERR_WORKSPACE : KDA_OK;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  kda::PrefillArgs a{q, k, v, g, beta, initial_state, o, final_state,
                     nck > 0 ? checkpoints : nullptr, B, T, H, checkpoint_every,
                     nseg > 1 ? seg_len : T, nseg, 0, nullptr, nullptr, nullptr,
                     n_ck > 0 ? ck_pos : nullptr, n_ck, gate_logits ? 1 : 0, ogate, nullptr};
#ifdef KDA_DEBUG_RANGE
  if (range_flags_address(&a.range_flags) != hipSuccess) return KDA_ERR_HIP;
#endif
  if (nseg > 1) {
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    float* seg_in = reinterpret_cast<float*>(ws);
    float* seg_z = reinterpret_cast<float*>(ws + off_z);
    float* seg_p = reinterpret_cast<float*>(ws + off_p);
    kda::PrefillArgs s1 = a;
    s1.mode = 1;
    s1.seg_z = seg_z;
    s1.seg_p = seg_p;
    hipError_t e;
    if (nseg >= 3 && kda::summary_split_ok(dk, dv, bf16, chunk)) {
      // segment 0 by the ordinary workgroups; the zero-start states and transitions of
      // segments 1 .. nseg-2 by the 128-column summary workgroups, in the same launch
      kda::PrefillArgs a0 = s1, a1 = s1;
      a0.seg_first = 0, a0.seg_count = 1, a0.with_p = 0;
      a1.seg_first = 1, a1.seg_count = nseg - 2, a1.with_p = 1;
      a1.ogate = nullptr;
      e = kda::chunk_fwd_summary(a0, a1, out == KDA_BF16, st);
    } else {
      e = launch_chunks(s1, chunk, dk, dv, bf16, out == KDA_BF16, st);
    }
    if (e == hipSuccess)
      e = kda::segment_scan(seg_z, seg_p, seg_in, B, H, nseg, dk, dv, st);
    if (e != hipSuccess) return KDA_ERR_HIP;
    a.seg_in = seg_in;
  }
  const hipError_t e = launch_chunks(a, chunk, dk, dv, bf16, out == KDA_BF16, st);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" int64_t kda_chunk_fwd_segment_tokens(int64_t B, int64_t T, int64_t H, int dk, int dv,
                                                int chunk, kda_dtype_t in) {
  if (!sizes_ok(B, T, H, dk, dv, chunk, in)) return 0;
  return auto_segment_tokens(B, T, H, dk, dv, in == KDA_BF16, chunk);
}

extern "C" size_t kda_chunk_fwd_segmented_workspace_bytes(int64_t B, int64_t T, int64_t H, int dk,
                                                          int dv, int chunk, kda_dtype_t in,
                                                          int64_t segment_tokens) {
  if (!sizes_ok(B, T, H, dk, dv, chunk, in) || segment_tokens < 1 || segment_tokens % chunk != 0)
    return 0;
  const int64_t nseg = num_segments(T, segment_tokens);
  if (!mul_ok(B * H, nseg) || !mul_ok(B * H * nseg, (int64_t)dk * (2 * dv + dk) * 4)) return 0;
  return segment_workspace(B, H, nseg, dk, dv, nullptr, nullptr);
}

extern "C" size_t kda_chunk_fwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int dk, int dv,
                                                int chunk, kda_dtype_t in) {
  if (!sizes_ok(B, T, H, dk, dv, chunk, in)) return 0;
  return kda_chunk_fwd_segmented_workspace_bytes(
      B, T, H, dk, dv, chunk, in, auto_segment_tokens(B, T, H, dk, dv, in == KDA_BF16, chunk));
}

extern "C" kda_status_t kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g,
                                      const void* beta, const float* initial_state, void* o,
                                      float* final_state, float* checkpoints,
                                      int64_t checkpoint_every, int64_t B, int64_t T, int64_t H,
                                      int dk, int dv, int chunk, kda_dtype_t in, kda_dtype_t out,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  const int64_t seg = sizes_ok(B, T, H, dk, dv, chunk, in)
                          ? auto_segment_tokens(B, T, H, dk, dv, in == KDA_BF16, chunk)
                          : kChunk;
  return chunk_fwd_impl(q, k, v, g, beta, initial_state, o, final_state, checkpoints,
                        checkpoint_every, B, T, H, dk, dv, chunk, in, out, seg, workspace,
                        workspace_bytes, stream);
}

extern "C" kda_status_t kda_chunk_fwd_segmented(
    const void* q, const void* k, const void* v, const void* g, const void* beta,
    const float* initial_state, void* o, float* final_state, float* checkpoints,
    int64_t checkpoint_every, int64_t B, int64_t T, int64_t H, int dk, int dv, int chunk,
    kda_dtype_t in, kda_dtype_t out, int64_t segment_tokens, void* workspace,
    size_t workspace_bytes, void* stream) {
  return chunk_fwd_impl(q, k, v, g, beta, initial_state, o, final_state, checkpoints,
                        checkpoint_every, B, T, H, dk, dv, chunk, in, out, segment_tokens,
                        workspace, workspace_bytes, stream);
}

static kda_status_t recurrent_step_impl(const void* q, const void* k, const void* v, const void* g,
                                        const void* beta, float* state, void* o, int64_t N,
                                        int64_t H, int dk, int dv, kda_dtype_t in, kda_dtype_t out,
                                        void* stream, bool gate_logits,
                                        const void* ogate = nullptr) {
  if (!q || !k || !v || !g || !beta || !state || !o) return KDA_ERR_NULL;
  if (!dtype_ok(in) || !dtype_ok(out)) return KDA_ERR_DTYPE;
  if (N < 1 || H < 1 || !head_dim_ok(dk) || !head_dim_ok(dv)) return KDA_ERR_SHAPE;
  if (!mul_ok(N, H) || N * H > INT32_MAX) return KDA_ERR_SHAPE;
  const void* ptrs[] = {q, k, v, g, beta, state, o};
  for (const void* p : ptrs)
    if (!aligned16(p)) return KDA_ERR_ALIGN;
  if (ogate && !aligned16(ogate)) return KDA_ERR_ALIGN;
  const int64_t nh = N * H, es = esize(in);
  const Span ss = span(state, nh * dk * dv * 4);
  const Span so = span(o, nh * dv * esize(out));
  const Span inputs[] = {span(q, nh * dk * es), span(k, nh * dk * es), span(v, nh * dv * es),
                         span(g, nh * dk * es), span(beta, nh * es),
                         ogate ? span(ogate, nh * dv * es) : Span{0, 0}};
  if (overlaps(so, ss)) return KDA_ERR_ALIAS;
  for (const Span& s : inputs)
    if (overlaps(so, s) || overlaps(ss, s)) return KDA_ERR_ALIAS;
  const hipError_t e = kda::decode_step(q, k, v, g, beta, state, o, nh, dk, dv, in == KDA_BF16,
                                        out == KDA_BF16, reinterpret_cast<hipStream_t>(stream),
                                        gate_logits, ogate);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

extern "C" kda_status_t kda_recurrent_step_output_gate(const void* q, const void* k,
                                                       const void* v, const void* g,
                                                       const void* beta, const void* gate,
                                                       float* state, void* o, int64_t N,
                                                       int64_t H, int dk, int dv, kda_dtype_t in,
                                                       kda_dtype_t out, void* stream) {
  if (!gate) return KDA_ERR_NULL;
  return recurrent_step_impl(q, k, v, g, beta, state, o, N, H, dk, dv, in, out, stream, false,
                             gate);
}

extern "C" kda_status_t kda_recurrent_step(const void* q, const void* k, const void* v,
                                           const void* g, const void* beta, float* state, void* o,
                                           int64_t N, int64_t H, int dk, int dv, kda_dtype_t in,
                                           kda_dtype_t out, void* stream) {
  return recurrent_step_impl(q, k, v, g, beta, state, o, N, H, dk, dv, in, out, stream, false);
}

extern "C" kda_status_t kda_recurrent_step_gate_logits(const void* q, const void* k, const void* v,
                                                       const void* a, const void* beta,
                                                       float* state, void* o, int64_t N,
                                                       int64_t H, int dk, int dv, kda_dtype_t in,
                                                       kda_dtype_t out, void* stream) {
  return recurrent_step_impl(q, k, v, a, beta, state, o, N, H, dk, dv, in, out, stream, true);
}

namespace {

kda_status_t multi_token_impl(const void* q, const void* k, const void* v, const void* g,
                              const void* beta, const int32_t* accept, float* state, void* o,
                              int64_t N, int64_t K, int64_t H, int dk, int dv, kda_dtype_t in,
                              kda_dtype_t out, bool commit, void* stream) {
  if (!k || !v || !g || !beta || !state) return KDA_ERR_NULL;
  if (commit ? !accept : (!q || !o)) return KDA_ERR_NULL;
  if (!dtype_ok(in) || !dtype_ok(out)) return KDA_ERR_DTYPE;
  if (commit && in != out) return KDA_ERR_DTYPE;  // commit reads no q and writes no o
  if (N < 1 || K < 1 || H < 1 || !head_dim_ok(dk) || !head_dim_ok(dv)) return KDA_ERR_SHAPE;
  if (!mul_ok(N, H) || N * H > INT32_MAX || !mul_ok(N * H, K) || !mul_ok(N * H * K, 128))
    return KDA_ERR_SHAPE;
  const void* ptrs[] = {q, k, v, g, beta, accept, state, o};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KDA_ERR_ALIGN;
  const int64_t nh = N * H, ntok = nh * K, es = esize(in);
  const Span ss = span(state, nh * dk * dv * 4);
  const Span inputs[] = {span(k, ntok * dk * es), span(v, ntok * dv * es), span(g, ntok * dk * es),
                         span(beta, ntok * es)};
  for (const Span& s : inputs)
    if (overlaps(ss, s)) return KDA_ERR_ALIAS;
  if (q && overlaps(ss, span(q, ntok * dk * es))) return KDA_ERR_ALIAS;
  if (commit && overlaps(ss, span(accept, N * 4))) return KDA_ERR_ALIAS;
  if (!commit) {
    const Span so = span(o, ntok * dv * esize(out));
    if (overlaps(so, ss) || overlaps(so, span(q, ntok * dk * es))) return KDA_ERR_ALIAS;
    for (const Span& s : inputs)
      if (overlaps(so, s)) return KDA_ERR_ALIAS;
  }
  const hipError_t e = kda::multi_token(q, k, v, g, beta, accept, state, o, N, K, H, dk, dv,
                                        in == KDA_BF16, out == KDA_BF16, commit,
                                        reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" kda_status_t kda_recurrent_verify(const void* q, const void* k, const void* v,
                                             const void* g, const void* beta, const float* state,
                                             void* o, int64_t N, int64_t K, int64_t H, int dk,
                                             int dv, kda_dtype_t in, kda_dtype_t out,
                                             void* stream) {
  return multi_token_impl(q, k, v, g, beta, nullptr, const_cast<float*>(state), o, N, K, H, dk,
                          dv, in, out, false, stream);
}

extern "C" kda_status_t kda_recurrent_commit(const void* k, const void* v, const void* g,
                                             const void* beta, const int32_t* accept,
                                             float* state, int64_t N, int64_t K, int64_t H,
                                             int dk, int dv, kda_dtype_t in, void* stream) {
  return multi_token_impl(nullptr, k, v, g, beta, accept, state, nullptr, N, K, H, dk, dv, in, in,
                          true, stream);
}

extern "C" kda_status_t kda_chunk_fwd_checkpoints_at(
    const void* q, const void* k, const void* v, const void* g, const void* beta,
    const float* initial_state, void* o, float* final_state, float* checkpoints,
    const int64_t* positions, int64_t n_positions, int64_t B, int64_t T, int64_t H, int dk, int dv,
    int chunk, kda_dtype_t in, kda_dtype_t out, void* workspace, size_t workspace_bytes,
    void* stream) {
  if (n_positions < 1) return KDA_ERR_SHAPE;
  const int64_t seg = sizes_ok(B, T, H, dk, dv, chunk, in)
                          ? auto_segment_tokens(B, T, H, dk, dv, in == KDA_BF16, chunk)
                          : kChunk;
  return chunk_fwd_impl(q, k, v, g, beta, initial_state, o, final_state, checkpoints, 0, B, T, H,
                        dk, dv, chunk, in, out, seg, workspace, workspace_bytes, stream, positions,
                        n_positions);
}

extern "C" kda_status_t kda_chunk_fwd_gate_logits(
    const void* q, const void* k, const void* v, const void* a, const void* beta,
    const float* initial_state, void* o, float* final_state, float* checkpoints,
    int64_t checkpoint_every, int64_t B, int64_t T, int64_t H, int dk, int dv, int chunk,
    kda_dtype_t in, kda_dtype_t out, void* workspace, size_t workspace_bytes, void* stream) {
  const int64_t seg = sizes_ok(B, T, H, dk, dv, chunk, in)
                          ? auto_segment_tokens(B, T, H, dk, dv, in == KDA_BF16, chunk)
                          : kChunk;
  return chunk_fwd_impl(q, k, v, a, beta, initial_state, o, final_state, checkpoints,
                        checkpoint_every, B, T, H, dk, dv, chunk, in, out, seg, workspace,
                        workspace_bytes, stream, nullptr, 0, true);
}

extern "C" kda_status_t kda_chunk_fwd_output_gate(
    const void* q, const void* k, const void* v, const void* g, const void* beta, const void* gate,
    const float* initial_state, void* o, float* final_state, float* checkpoints,
    int64_t checkpoint_every, int64_t B, int64_t T, int64_t H, int dk, int dv, int chunk,
    kda_dtype_t in, kda_dtype_t out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!gate) return KDA_ERR_NULL;
  const int64_t seg = sizes_ok(B, T, H, dk, dv, chunk, in)
                          ? auto_segment_tokens(B, T, H, dk, dv, in == KDA_BF16, chunk)
                          : kChunk;
  return chunk_fwd_impl(q, k, v, g, beta, initial_state, o, final_state, checkpoints,
                        checkpoint_every, B, T, H, dk, dv, chunk, in, out, seg, workspace,
                        workspace_bytes, stream, nullptr, 0, false, gate);
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// Device address of the scratch array on the current device, looked up once per
// device (with that device current) and kept.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" kda_status_t kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                              const void* g, const void* beta,
                                              const float* initial_state, void* o,
                                              float* final_state, float* checkpoints,
                                              int64_t checkpoint_every, int64_t B, int64_t T,
                                              int64_t H, int dk, int dv, int chunk,
                                              kda_dtype_t in, kda_dtype_t out, void* stream) {
  if (!sizes_ok(B, T, H, dk, dv, chunk, in)) return KDA_ERR_SHAPE;
  const int64_t seg = auto_segment_tokens(B, T, H, dk, dv, in == KDA_BF16, chunk);
  const int64_t nseg = num_segments(T, seg);
  if (!mul_ok(B * H, nseg) || !mul_ok(B * H * nseg, (int64_t)dk * (2 * dv + dk) * 4))
    return KDA_ERR_SHAPE;
  const size_t need = segment_workspace(B, H, nseg, dk, dv, nullptr, nullptr);
  if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    // the other arguments are checked first, so that a bad call touches no GPU state
    const kda_status_t st0 =
        chunk_fwd_impl(q, k, v, g, beta, initial_state, o, final_state, checkpoints,
                       checkpoint_every, B, T, H, dk, dv, chunk, in, out, seg, nullptr, 0,
                       stream, nullptr, 0, false, nullptr, /*validate_only=*/true);
    if (st0 != KDA_ERR_WORKSPACE) return st0;
    if (scratch_address(&ws) != hipSuccess) return KDA_ERR_HIP;
  }
  return chunk_fwd_impl(q, k, v, g, beta, initial_state, o, final_state, checkpoints,
                        checkpoint_every, B, T, H, dk, dv, chunk, in, out, seg, ws,
                        ws ? (size_t)KDA_NOALLOC_SCRATCH_BYTES : 0, stream);
}

#ifdef KDA_DEBUG_RANGE
extern "C" kda_status_t kda_debug_range_flags(unsigned* flags, int clear) {
  if (!flags) return KDA_ERR_NULL;
  unsigned* p = nullptr;
  if (range_flags_address(&p) != hipSuccess) return KDA_ERR_HIP;
  if (hipMemcpy(flags, p, sizeof(unsigned), hipMemcpyDeviceToHost) != hipSuccess)
    return KDA_ERR_HIP;
  if (clear) {
    const unsigned zero = 0u;
    if (hipMemcpy(p, &zero, sizeof(unsigned), hipMemcpyHostToDevice) != hipSuccess)
      return KDA_ERR_HIP;
  }
  return KDA_OK;
}
#endif
