// Host side of the C ABI declared in include/kda.h: argument validation,
// dispatch to the gfx950 kernels, status codes.  Nothing here allocates device
// memory or synchronises.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "kda.h"
#include "kda_internal.h"


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
  }
  return "KDA_ERR_UNKNOWN";
}

extern "C" size_t kda_chunk_fwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int dk, int dv,
                                                int chunk, kda_dtype_t in) {
  (void)B;
  (void)T;
  (void)H;
  (void)dk;
  (void)dv;
  (void)chunk;
  (void)in;
  return 0;  // the fused kernel keeps every intermediate on chip
}

extern "C" kda_status_t kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g,
                                      const void* beta, const float* initial_state, void* o,
                                      float* final_state, float* checkpoints,
                                      int64_t checkpoint_every, int64_t B, int64_t T, int64_t H,
                                      int dk, int dv, int chunk, kda_dtype_t in, kda_dtype_t out,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (!q || !k || !v || !g || !beta || !o) return KDA_ERR_NULL;
  if (checkpoint_every != 0 && !checkpoints) return KDA_ERR_NULL;
  if (!dtype_ok(in) || !dtype_ok(out)) return KDA_ERR_DTYPE;
  if (B < 1 || T < 1 || H < 1 || !head_dim_ok(dk) || !head_dim_ok(dv) || chunk != 64)
    return KDA_ERR_SHAPE;
  if (in == KDA_F32 && (dk != 64 || dv != 64)) return KDA_ERR_SHAPE;
  if (checkpoint_every < 0 || (checkpoint_every % chunk) != 0) return KDA_ERR_SHAPE;
  if (!mul_ok(B, T) || !mul_ok(B * T, H) || !mul_ok(B * T * H, 128)) return KDA_ERR_SHAPE;
  const int64_t heads = B * H;
  if (kda::prefill_grid(heads, dk, dv, in == KDA_BF16) > INT32_MAX) return KDA_ERR_SHAPE;

  const void* ptrs[] = {q, k, v, g, beta, initial_state, o, final_state, checkpoints};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KDA_ERR_ALIGN;

  const int64_t es = esize(in);
  const int64_t ntok = B * T * H;
  const Span sq = span(q, ntok * dk * es), sk = span(k, ntok * dk * es);
  const Span sv = span(v, ntok * dv * es), sg = span(g, ntok * dk * es);
  const Span sb = span(beta, ntok * es);
  const Span so = span(o, ntok * dv * esize(out));
  const int64_t state_bytes = heads * dk * dv * 4;
  const Span inputs[] = {sq, sk, sv, sg, sb};
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
  if (checkpoints) {
    const int64_t nck = T / checkpoint_every;
    const Span sc = span(checkpoints, B * nck * H * dk * dv * 4);
    if (overlaps(sc, so)) return KDA_ERR_ALIAS;
    for (const Span& s : inputs)
      if (overlaps(sc, s)) return KDA_ERR_ALIAS;
    if (initial_state && overlaps(sc, span(initial_state, state_bytes))) return KDA_ERR_ALIAS;
    if (final_state && overlaps(sc, span(final_state, state_bytes))) return KDA_ERR_ALIAS;
  }

  kda::PrefillArgs a{q, k, v, g, beta, initial_state, o, final_state,
                     checkpoint_every ? checkpoints : nullptr, B, T, H, checkpoint_every};
  const hipError_t e = kda::chunk_fwd(a, dk, dv, in == KDA_BF16, out == KDA_BF16,
                                      reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

extern "C" kda_status_t kda_recurrent_step(const void* q, const void* k, const void* v,
                                           const void* g, const void* beta, float* state, void* o,
                                           int64_t N, int64_t H, int dk, int dv, kda_dtype_t in,
                                           kda_dtype_t out, void* stream) {
  if (!q || !k || !v || !g || !beta || !state || !o) return KDA_ERR_NULL;
  if (!dtype_ok(in) || !dtype_ok(out)) return KDA_ERR_DTYPE;
  if (N < 1 || H < 1 || !head_dim_ok(dk) || !head_dim_ok(dv)) return KDA_ERR_SHAPE;
  if (!mul_ok(N, H) || N * H > INT32_MAX) return KDA_ERR_SHAPE;
  const void* ptrs[] = {q, k, v, g, beta, state, o};
  for (const void* p : ptrs)
    if (!aligned16(p)) return KDA_ERR_ALIGN;
  const int64_t nh = N * H, es = esize(in);
  const Span ss = span(state, nh * dk * dv * 4);
  const Span so = span(o, nh * dv * esize(out));
  const Span inputs[] = {span(q, nh * dk * es), span(k, nh * dk * es), span(v, nh * dv * es),
                         span(g, nh * dk * es), span(beta, nh * es)};
  if (overlaps(so, ss)) return KDA_ERR_ALIAS;
  for (const Span& s : inputs)
    if (overlaps(so, s) || overlaps(ss, s)) return KDA_ERR_ALIAS;
  const hipError_t e = kda::decode_step(q, k, v, g, beta, state, o, nh, dk, dv, in == KDA_BF16,
                                        out == KDA_BF16, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}
