// Internal interface between the C-ABI host code and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

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
};

// Number of workgroups the prefill launch uses for B*H heads (fits int32 or not).
int64_t prefill_grid(int64_t heads, int dk, int dv, bool in_bf16);

hipError_t chunk_fwd(const PrefillArgs& a, int dk, int dv, bool in_bf16, bool out_bf16,
                     hipStream_t s);

hipError_t decode_step(const void* q, const void* k, const void* v, const void* g,
                       const void* beta, float* state, void* o, int64_t nh, int dk, int dv,
                       bool in_bf16, bool out_bf16, hipStream_t s);

}  // namespace kda
