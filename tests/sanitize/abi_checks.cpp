// Host-side argument validation of the C ABI (include/kda.h), for a build whose host
// code carries AddressSanitizer and UndefinedBehaviorSanitizer.  Every call below is
// one the library must reject before anything is enqueued, or a pure size query, so
// no GPU is needed and none is touched.  The pointers are addresses inside one host
// pool: validation compares them (alignment, overlaps) but never dereferences them.
// Extreme sizes drive the size arithmetic (element counts, byte spans, workspace
// sizes, segment lengths) to its limits, where an overflow would be undefined
// behaviour that the sanitizer reports.
//
// Exit status 0 when every call returns the expected status; the sanitizers abort on
// their first report.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include "kda.h"

namespace {

int g_failures = 0;
int g_checks = 0;

void expect(const char* what, int got, int want) {
  ++g_checks;
  if (got != want) {
    ++g_failures;
    printf("FAIL %s: got %d (%s), want %d (%s)\n", what, got,
           kda_status_str(static_cast<kda_status_t>(got)), want,
           kda_status_str(static_cast<kda_status_t>(want)));
  }
}

void expect_true(const char* what, bool ok) {
  ++g_checks;
  if (!ok) {
    ++g_failures;
    printf("FAIL %s\n", what);
  }
}

alignas(256) unsigned char g_pool[32 << 16];

// distinct 16-byte aligned host addresses, 64 KiB apart (one d = 128 state each)
void* P(int i) { return g_pool + (65536 * i); }
float* F(int i) { return reinterpret_cast<float*>(P(i)); }

const kda_dtype_t BF = KDA_BF16, F32 = KDA_F32;

// kda_chunk_fwd with defaults that pass validation up to the point a case changes
struct Fwd {
  const void *q = P(1), *k = P(2), *v = P(3), *g = P(4), *beta = P(5);
  const float* s0 = nullptr;
  void* o = P(6);
  float *sf = nullptr, *ck = nullptr;
  int64_t every = 0, B = 1, T = 256, H = 2;
  int dk = 128, dv = 128, chunk = 64;
  kda_dtype_t in = BF, out = BF;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  int run() const {
    return kda_chunk_fwd(q, k, v, g, beta, s0, o, sf, ck, every, B, T, H, dk, dv, chunk, in,
                         out, ws, ws_bytes, nullptr);
  }
  int run_segmented(int64_t seg) const {
    return kda_chunk_fwd_segmented(q, k, v, g, beta, s0, o, sf, ck, every, B, T, H, dk, dv,
                                   chunk, in, out, seg, ws, ws_bytes, nullptr);
  }
  int run_noalloc() const {
    return kda_chunk_fwd_noalloc(q, k, v, g, beta, s0, o, sf, ck, every, B, T, H, dk, dv, chunk,
                                 in, out, nullptr);
  }
  int run_gate(const void* z) const {
    return kda_chunk_fwd_output_gate(q, k, v, g, beta, z, s0, o, sf, ck, every, B, T, H, dk, dv,
                                     chunk, in, out, ws, ws_bytes, nullptr);
  }
  int run_logits() const {
    return kda_chunk_fwd_gate_logits(q, k, v, g, beta, s0, o, sf, ck, every, B, T, H, dk, dv,
                                     chunk, in, out, ws, ws_bytes, nullptr);
  }
  int run_at(const int64_t* pos, int64_t n) const {
    return kda_chunk_fwd_checkpoints_at(q, k, v, g, beta, s0, o, sf, ck, pos, n, B, T, H, dk, dv,
                                        chunk, in, out, ws, ws_bytes, nullptr);
  }
};

void status_strings() {
  const int codes[] = {KDA_OK,            KDA_ERR_NULL,  KDA_ERR_SHAPE, KDA_ERR_DTYPE,
                       KDA_ERR_ALIGN,     KDA_ERR_WORKSPACE, KDA_ERR_ALIAS, KDA_ERR_HIP,
                       -99,               99};
  for (int c : codes) {
    const char* s = kda_status_str(static_cast<kda_status_t>(c));
    expect_true("status string not NULL", s != nullptr && strncmp(s, "KDA_", 4) == 0);
  }
}

void size_queries() {
  const int64_t big = INT64_MAX;
  // unsupported or overflowing sizes: 0
  expect_true("ws: dk 96", kda_chunk_fwd_workspace_bytes(1, 256, 2, 96, 128, 64, BF) == 0);
  expect_true("ws: chunk 32 f32", kda_chunk_fwd_workspace_bytes(1, 256, 2, 64, 64, 32, F32) == 0);
  expect_true("ws: B overflow", kda_chunk_fwd_workspace_bytes(big, big, big, 128, 128, 64, BF) == 0);
  expect_true("ws: T overflow", kda_chunk_fwd_workspace_bytes(1, big, 1, 128, 128, 64, BF) == 0);
  expect_true("seg: B overflow", kda_chunk_fwd_segment_tokens(big, 2, big, 128, 128, 64, BF) == 0);
  expect_true("seg: H bound", kda_chunk_fwd_segment_tokens(1, 64, 131072, 128, 128, 64, BF) == 0);
  expect_true("segws: seg 0",
              kda_chunk_fwd_segmented_workspace_bytes(1, 4096, 2, 128, 128, 64, BF, 0) == 0);
  expect_true("segws: seg 100",
              kda_chunk_fwd_segmented_workspace_bytes(1, 4096, 2, 128, 128, 64, BF, 100) == 0);
  // supported sizes: few heads on a long sequence take segments and a workspace
  expect_true("ws: few heads", kda_chunk_fwd_workspace_bytes(1, 65536, 32, 128, 128, 64, BF) > 0);
  expect_true("ws: many heads", kda_chunk_fwd_workspace_bytes(4, 4096, 32, 128, 128, 64, BF) == 0);
  const int64_t seg = kda_chunk_fwd_segment_tokens(1, 1 << 20, 16, 128, 128, 64, BF);
  expect_true("seg: multiple of 64", seg > 0 && seg % 64 == 0 && seg < (1 << 20));
  // the longest sequences the size checks admit: the segment model and the
  // workspace arithmetic stay defined
  for (int64_t t : {(int64_t)1 << 40, (int64_t)1 << 52, (int64_t)1 << 54}) {
    const int64_t s = kda_chunk_fwd_segment_tokens(1, t, 1, 128, 128, 64, BF);
    const size_t w = kda_chunk_fwd_workspace_bytes(1, t, 1, 128, 128, 64, BF);
    expect_true("long T: segment length", s == 0 || s % 64 == 0);
    (void)w;
  }
  for (int c : {16, 32, 64})
    expect_true("segws: chunk",
                kda_chunk_fwd_segmented_workspace_bytes(1, 4096, 2, 128, 128, c, BF, 1024) > 0);
}

void chunk_fwd_cases() {
  Fwd a;
  {
    Fwd x = a;
    x.q = nullptr;
    expect("fwd q NULL", x.run(), KDA_ERR_NULL);
  }
  {
    Fwd x = a;
    x.every = 64;
    expect("fwd checkpoints NULL", x.run(), KDA_ERR_NULL);
  }
  {
    Fwd x = a;
    x.in = static_cast<kda_dtype_t>(5);
    expect("fwd dtype", x.run(), KDA_ERR_DTYPE);
  }
  {
    Fwd x = a;
    x.out = static_cast<kda_dtype_t>(-1);
    expect("fwd out dtype", x.run(), KDA_ERR_DTYPE);
  }
  for (int d : {0, 32, 96, 256}) {
    Fwd x = a;
    x.dk = d;
    expect("fwd dk", x.run(), KDA_ERR_SHAPE);
    x = a;
    x.dv = d;
    expect("fwd dv", x.run(), KDA_ERR_SHAPE);
  }
  for (int c : {0, -64, 1, 8, 48, 128}) {
    Fwd x = a;
    x.chunk = c;
    expect("fwd chunk", x.run(), KDA_ERR_SHAPE);
  }
  {
    Fwd x = a;
    x.in = x.out = F32;
    x.dk = x.dv = 64;
    x.chunk = 32;
    expect("fwd chunk 32 f32", x.run(), KDA_ERR_SHAPE);
    x.dk = x.dv = 128;
    x.chunk = 64;
    expect("fwd f32 d128", x.run(), KDA_ERR_SHAPE);
  }
  for (int64_t t : {(int64_t)0, (int64_t)-1, INT64_MIN}) {
    Fwd x = a;
    x.T = t;
    expect("fwd T", x.run(), KDA_ERR_SHAPE);
    x = a;
    x.B = t;
    expect("fwd B", x.run(), KDA_ERR_SHAPE);
    x = a;
    x.H = t;
    expect("fwd H", x.run(), KDA_ERR_SHAPE);
  }
  {
    // the 32-bit row offsets: H = 131,072 at d = 128 is rejected; 131,071 passes the
    // size check and is stopped by the misaligned q
    Fwd x = a;
    x.T = 1;
    x.H = 131072;
    expect("fwd H bound", x.run(), KDA_ERR_SHAPE);
    x.H = 131071;
    x.q = static_cast<const unsigned char*>(P(1)) + 8;
    expect("fwd H at bound", x.run(), KDA_ERR_ALIGN);
  }
  {
    // element counts and byte spans at the edge of int64
    const int64_t big = INT64_MAX;
    for (int64_t t : {(int64_t)1 << 55, (int64_t)1 << 56, (int64_t)1 << 60, big}) {
      Fwd x = a;
      x.T = t;
      x.H = 1;
      x.ws = P(9);
      x.ws_bytes = SIZE_MAX;
      const int st = x.run();
      expect_true("fwd huge T rejected", st == KDA_ERR_SHAPE);
    }
    Fwd x = a;
    x.B = big;
    x.T = big;
    expect("fwd B*T overflow", x.run(), KDA_ERR_SHAPE);
  }
  for (int64_t e : {(int64_t)-64, (int64_t)1, (int64_t)100, (int64_t)32}) {
    Fwd x = a;
    x.every = e;
    x.ck = F(8);
    expect("fwd checkpoint_every", x.run(), KDA_ERR_SHAPE);
  }
  {
    Fwd x = a;
    x.q = static_cast<const unsigned char*>(P(1)) + 8;
    expect("fwd q misaligned", x.run(), KDA_ERR_ALIGN);
    x = a;
    x.sf = reinterpret_cast<float*>(static_cast<unsigned char*>(P(7)) + 4);
    expect("fwd final misaligned", x.run(), KDA_ERR_ALIGN);
  }
  {
    // overlaps: o with an input, the final state with o or (partly) the initial state,
    // checkpoints with the final state
    Fwd x = a;
    x.o = const_cast<void*>(x.v);
    expect("fwd o == v", x.run(), KDA_ERR_ALIAS);
    x = a;
    x.B = 1;
    x.T = 1;
    x.H = 1;
    x.o = static_cast<unsigned char*>(const_cast<void*>(x.q)) + 128;  // inside q's 256 bytes
    expect("fwd o inside q", x.run(), KDA_ERR_ALIAS);
    x = a;
    x.sf = reinterpret_cast<float*>(x.o);
    expect("fwd final == o", x.run(), KDA_ERR_ALIAS);
    x = a;
    x.T = 1;
    x.H = 1;
    x.s0 = F(10);
    x.sf = reinterpret_cast<float*>(static_cast<unsigned char*>(P(10)) + 16);
    expect("fwd final partly initial", x.run(), KDA_ERR_ALIAS);
    x = a;
    x.T = 64;
    x.H = 1;
    x.every = 64;
    x.sf = F(11);
    x.ck = F(11);
    expect("fwd checkpoints == final", x.run(), KDA_ERR_ALIAS);
  }
}

void segment_cases() {
  Fwd a;
  for (int64_t s : {(int64_t)0, (int64_t)-64, (int64_t)100, (int64_t)32}) {
    expect("seg length", a.run_segmented(s), KDA_ERR_SHAPE);
  }
  {
    // several segments need a workspace: missing, too small, overlapping
    expect("seg ws missing", a.run_segmented(64), KDA_ERR_WORKSPACE);
    Fwd x = a;
    x.ws = P(12);
    x.ws_bytes = 16;
    expect("seg ws small", x.run_segmented(64), KDA_ERR_WORKSPACE);
    x.ws = const_cast<void*>(x.k);
    x.ws_bytes = SIZE_MAX / 4;
    expect("seg ws overlaps k", x.run_segmented(64), KDA_ERR_ALIAS);
  }
  {
    // few heads, long sequence: the library's own segmentation needs a workspace
    Fwd x = a;
    x.T = 65536;
    x.H = 32;
    expect("auto seg ws missing", x.run(), KDA_ERR_WORKSPACE);
    expect("noalloc: q NULL", (x.q = nullptr, x.run_noalloc()), KDA_ERR_NULL);
    x.q = static_cast<const unsigned char*>(P(1)) + 4;
    expect("noalloc: q misaligned", x.run_noalloc(), KDA_ERR_ALIGN);
    x.q = P(1);
    x.o = const_cast<void*>(x.g);
    expect("noalloc: o == g", x.run_noalloc(), KDA_ERR_ALIAS);
  }
  {
    // the segment workspace the library picks, over batch, heads and lengths: it fits
    // the no-allocation entry point's static array
    size_t most = 0;
    for (int64_t b : {1, 2, 4})
      for (int64_t h = 1; h <= 128; h *= 2)
        for (int64_t t = (int64_t)1 << 12; t <= ((int64_t)1 << 30); t <<= 2)
          for (int c : {16, 32, 64}) {
            const size_t w = kda_chunk_fwd_workspace_bytes(b, t, h, 128, 128, c, BF);
            most = w > most ? w : most;
          }
    printf("largest automatic segment workspace: %zu bytes\n", most);
    expect_true("automatic workspace fits the static array",
                most > 0 && most <= (size_t)KDA_NOALLOC_SCRATCH_BYTES);
  }
  {
    Fwd x = a;
    x.dk = 96;
    expect("noalloc: dk", x.run_noalloc(), KDA_ERR_SHAPE);
    x = a;
    x.chunk = 48;
    expect("noalloc: chunk", x.run_noalloc(), KDA_ERR_SHAPE);
  }
}

void variant_cases() {
  Fwd a;
  expect("gate NULL", a.run_gate(nullptr), KDA_ERR_NULL);
  expect("gate misaligned", a.run_gate(static_cast<unsigned char*>(P(13)) + 2), KDA_ERR_ALIGN);
  expect("gate == o", a.run_gate(a.o), KDA_ERR_ALIAS);
  {
    Fwd x = a;
    x.beta = nullptr;
    expect("logits beta NULL", x.run_logits(), KDA_ERR_NULL);
    x = a;
    x.chunk = 16;
    x.in = x.out = F32;
    x.dk = x.dv = 64;
    expect("logits chunk 16 f32", x.run_logits(), KDA_ERR_SHAPE);
  }
  alignas(16) static int64_t pos[4] = {64, 128, 192, 256};
  expect("at: n 0", a.run_at(pos, 0), KDA_ERR_SHAPE);
  expect("at: n -1", a.run_at(pos, -1), KDA_ERR_SHAPE);
  expect("at: positions NULL", (Fwd(a).run_at(nullptr, 3)), KDA_ERR_NULL);
  {
    Fwd x = a;
    x.ck = F(14);
    expect("at: positions NULL", x.run_at(nullptr, 3), KDA_ERR_NULL);
    expect("at: positions misaligned",
           x.run_at(reinterpret_cast<const int64_t*>(reinterpret_cast<const char*>(pos) + 4), 3),
           KDA_ERR_ALIGN);
    x.ck = reinterpret_cast<float*>(x.o);
    expect("at: checkpoints == o", x.run_at(pos, 4), KDA_ERR_ALIAS);
  }
}

void decode_cases() {
  const void *q = P(1), *k = P(2), *v = P(3), *g = P(4), *beta = P(5), *z = P(7);
  float* st = F(8);
  void* o = P(6);
  expect("step state NULL", kda_recurrent_step(q, k, v, g, beta, nullptr, o, 4, 2, 128, 128, BF, BF, nullptr),
         KDA_ERR_NULL);
  expect("step dtype", kda_recurrent_step(q, k, v, g, beta, st, o, 4, 2, 128, 128, BF,
                                          static_cast<kda_dtype_t>(3), nullptr),
         KDA_ERR_DTYPE);
  for (int64_t n : {(int64_t)0, (int64_t)-5})
    expect("step N", kda_recurrent_step(q, k, v, g, beta, st, o, n, 2, 128, 128, BF, BF, nullptr),
           KDA_ERR_SHAPE);
  expect("step N*H > int32", kda_recurrent_step(q, k, v, g, beta, st, o, (int64_t)1 << 20,
                                                (int64_t)1 << 12, 128, 128, BF, BF, nullptr),
         KDA_ERR_SHAPE);
  expect("step N*H overflow", kda_recurrent_step(q, k, v, g, beta, st, o, INT64_MAX, INT64_MAX,
                                                 128, 128, BF, BF, nullptr),
         KDA_ERR_SHAPE);
  expect("step dk", kda_recurrent_step(q, k, v, g, beta, st, o, 4, 2, 48, 128, BF, BF, nullptr),
         KDA_ERR_SHAPE);
  expect("step misaligned", kda_recurrent_step(q, k, v, g, static_cast<const char*>(beta) + 2, st,
                                               o, 4, 2, 128, 128, BF, BF, nullptr),
         KDA_ERR_ALIGN);
  expect("step o in state", kda_recurrent_step(q, k, v, g, beta, st, F(8) + 64, 1, 1, 128, 128,
                                               BF, BF, nullptr),
         KDA_ERR_ALIAS);
  expect("step state over k", kda_recurrent_step(q, k, v, g, beta, F(2), o, 1, 1, 64, 64, BF,
                                                 BF, nullptr),
         KDA_ERR_ALIAS);
  expect("step gate NULL", kda_recurrent_step_output_gate(q, k, v, g, beta, nullptr, st, o, 4, 2,
                                                         128, 128, BF, BF, nullptr),
         KDA_ERR_NULL);
  expect("step gate == o", kda_recurrent_step_output_gate(q, k, v, g, beta, o, st, o, 1, 1, 64,
                                                         64, BF, BF, nullptr),
         KDA_ERR_ALIAS);
  expect("step gate misaligned",
         kda_recurrent_step_output_gate(q, k, v, g, beta, static_cast<const char*>(z) + 8, st, o,
                                        1, 1, 64, 64, BF, BF, nullptr),
         KDA_ERR_ALIGN);
  expect("step logits NULL", kda_recurrent_step_gate_logits(q, k, v, nullptr, beta, st, o, 4, 2,
                                                           128, 128, BF, BF, nullptr),
         KDA_ERR_NULL);

  // speculative verify / commit
  alignas(16) static int32_t accept[4] = {1, 2, 3, 4};
  const float* cst = st;
  expect("verify q NULL", kda_recurrent_verify(nullptr, k, v, g, beta, cst, o, 4, 4, 2, 128, 128,
                                               BF, BF, nullptr),
         KDA_ERR_NULL);
  for (int64_t kk : {(int64_t)0, (int64_t)-1})
    expect("verify K", kda_recurrent_verify(q, k, v, g, beta, cst, o, 4, kk, 2, 128, 128, BF, BF,
                                            nullptr),
           KDA_ERR_SHAPE);
  expect("verify N*H*K overflow",
         kda_recurrent_verify(q, k, v, g, beta, cst, o, 1 << 20, INT64_MAX / 2, 1 << 10, 128, 128,
                              BF, BF, nullptr),
         KDA_ERR_SHAPE);
  expect("verify o over q", kda_recurrent_verify(q, k, v, g, beta, cst, const_cast<void*>(q), 1, 1,
                                                 1, 64, 64, BF, BF, nullptr),
         KDA_ERR_ALIAS);
  expect("commit accept NULL", kda_recurrent_commit(k, v, g, beta, nullptr, st, 4, 4, 2, 128, 128,
                                                    BF, nullptr),
         KDA_ERR_NULL);
  expect("commit accept misaligned",
         kda_recurrent_commit(k, v, g, beta,
                              reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(accept) + 4),
                              st, 4, 4, 2, 128, 128, BF, nullptr),
         KDA_ERR_ALIGN);
  expect("commit state over v", kda_recurrent_commit(k, v, g, beta, accept, F(3), 1, 1, 1, 64, 64,
                                                     BF, nullptr),
         KDA_ERR_ALIAS);
  expect("commit dtype", kda_recurrent_commit(k, v, g, beta, accept, st, 4, 4, 2, 128, 128,
                                              static_cast<kda_dtype_t>(9), nullptr),
         KDA_ERR_DTYPE);
}

}  // namespace

int main() {
  status_strings();
  size_queries();
  chunk_fwd_cases();
  segment_cases();
  variant_cases();
  decode_cases();
  printf("%d checks, %d failures\n", g_checks, g_failures);
  return g_failures == 0 ? 0 : 1;
}
