// Device-side helpers shared by the KDA kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
// Log-decay floor: each step keeps at least exp(-5) ~ 0.67% of a key channel
// (orkas.ai blog "Kimi K3 architecture", "A lower bound that deleted a GPU code
// path").
constexpr float kLogDecayFloor = -5.0f;

// min(max(g, -5), 0) that keeps NaN (fmaxf/fminf would drop it).
__device__ __forceinline__ float clamp_log_decay(float g) {
  // median of three: one instruction, no NaN canonicalisation; NaN passed through
  return (g != g) ? g : __builtin_amdgcn_fmed3f(g, kLogDecayFloor, 0.0f);
}

// Log-decay in base-2 units from a raw decay logit a: clamp(-softplus(a)) * log2(e),
// with -softplus(a) = -log2(1 + 2^(a log2 e)) / log2(e) (the negative-softplus map of
// the Towards-AI article on Kimi K3, "Kimi Delta Attention (KDA)").  For a above ~88
// 2^(...) overflows to +inf and the result is the floor, as it should be; NaN stays
// NaN.  In float32 1 + 2^t rounds away 2^t < 2^-24, i.e. log-decays above -6e-8
// become 0 (a relative decay error below 1e-7).
__device__ __forceinline__ float gamma_from_logit(float a) {
  const float t = -__builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(a * kLog2e));
  return (a != a) ? a : __builtin_amdgcn_fmed3f(t, kLogDecayFloor * kLog2e, 0.0f);
}

// ---- Range checks of the chunked forms (compiled in with -DKDA_DEBUG_RANGE only).
// The -5 floor bounds a 16-token sub-tile's cumulative decay, so a diagonal tile's row
// factor 2^L (L the inclusive log2-decay sum from the sub-tile's start) lies in
// [e^-80, 1] and its column factor 2^-L in [1, e^80] (orkas.ai blog "Kimi K3
// architecture", "A lower bound that deleted a GPU code path"), and every bfloat16
// operand is then finite for moderate key norms.  A debug build checks the factors,
// every operand, every kept A / P tile entry and the state after each chunk, and ORs
// one bit per kind of violation into a device word; a release build compiles the
// checks away.
enum : unsigned {
  kRangeFactor = 1u,   // a row factor outside [0, 1] or a column factor outside [1, e^80]
  kRangeOperand = 2u,  // an operand not finite or beyond the bfloat16 range
  kRangeTile = 4u,     // a kept entry of an A or P tile not finite
  kRangeState = 8u,    // a state value not finite after a chunk
};
constexpr float kE80 = 5.5406224e34f;        // e^80
constexpr float kBf16Max = 3.3895314e38f;    // largest finite bfloat16
struct RangeCheck {
  unsigned* flags;  // device word; NULL (or a release build): no checks
#ifdef KDA_DEBUG_RANGE
  __device__ __forceinline__ void operator()(bool bad, unsigned bit) const {
    if (bad && flags) atomicOr(flags, bit);
  }
  // row factor 2^L in [0, 1], column factor 2^-L in [1, e^80] (one rounding of slack)
  __device__ __forceinline__ void factors(float row, float col) const {
    (*this)(!(row >= 0.f && row <= 1.f), kRangeFactor);
    (*this)(!(col >= 0.99999f && col <= kE80 * 1.00001f), kRangeFactor);
  }
  __device__ __forceinline__ void operand(float x, float lim) const {
    (*this)(!(__builtin_fabsf(x) <= lim), kRangeOperand);
  }
  __device__ __forceinline__ void finite(float x, unsigned bit) const {
    (*this)(!(__builtin_fabsf(x) <= 3.4028235e38f), bit);
  }
#else
  __device__ __forceinline__ void operator()(bool, unsigned) const {}
  __device__ __forceinline__ void factors(float, float) const {}
  __device__ __forceinline__ void operand(float, float) const {}
  __device__ __forceinline__ void finite(float, unsigned) const {}
#endif
};

// 2^x on the hardware transcendental unit.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Logistic sigmoid 1 / (1 + e^-z) of the output gate, from 2^x and a reciprocal on the
// transcendental unit: z -> +inf gives 1, z -> -inf gives 0 (1 / inf), NaN stays NaN.
__device__ __forceinline__ float sigmoid_hw(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// Two adjacent elements in one register: a bfloat16 pair (low half = lower
// address) or a float32 pair.  pack2 rounds to nearest even.
__device__ __forceinline__ uint32_t pack2(f32x2 x, uint32_t*) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}
__device__ __forceinline__ f32x2 pack2(f32x2 x, f32x2*) { return x; }
__device__ __forceinline__ f32x2 unpack2(uint32_t u) {
  return f32x2{__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u)};
}
__device__ __forceinline__ f32x2 unpack2(f32x2 x) { return x; }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// Load 8 consecutive elements (16 bytes for bf16, 32 bytes for f32) as floats.
__device__ __forceinline__ void load8(const __bf16* p, float* out) {
  bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = (float)v[i];
}
__device__ __forceinline__ void load8(const float* p, float* out) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[i] = a[i];
    out[4 + i] = b[i];
  }
}

// 16 bytes of global input as floats: 8 bfloat16 or 4 float32 values.
__device__ __forceinline__ void load16(const __bf16* p, float* out) { load8(p, out); }
__device__ __forceinline__ void load16(const float* p, float* out) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = a[i];
}

__device__ __forceinline__ void store8(float* p, const float* x) {
  *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}

// Unpack 16 raw bytes held in a float4 register into floats (8 bfloat16 or 4
// float32 values) with bit operations only, so the register never goes to memory.
__device__ __forceinline__ void unpack16(const float4& raw, __bf16*, float* out) {
  const uint32_t w[4] = {__float_as_uint(raw.x), __float_as_uint(raw.y), __float_as_uint(raw.z),
                         __float_as_uint(raw.w)};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack16(const float4& raw, float*, float* out) {
  out[0] = raw.x;
  out[1] = raw.y;
  out[2] = raw.z;
  out[3] = raw.w;
}

__device__ __forceinline__ uint4 mask4(const float4& x, uint32_t m) {
  return make_uint4(__float_as_uint(x.x) & m, __float_as_uint(x.y) & m, __float_as_uint(x.z) & m,
                    __float_as_uint(x.w) & m);
}

// Access at a uniform base plus a 32-bit byte offset: this form lets the backend
// use the scalar-base addressing mode (SGPR base + one VGPR offset) instead of
// a 64-bit address per lane.
template <typename T>
__device__ __forceinline__ T ld_at(const void* base, uint32_t byte_off) {
  return *reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + byte_off);
}
template <typename T>
__device__ __forceinline__ void st_at(void* base, uint32_t byte_off, T x) {
  *reinterpret_cast<T*>(reinterpret_cast<char*>(base) + byte_off) = x;
}

// Wave-wide sum (64 lanes).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

}  // namespace kda
