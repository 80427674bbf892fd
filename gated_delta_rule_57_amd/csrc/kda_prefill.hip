// Chunked KDA forward (prefill): one workgroup per (batch row, head, d_v slice)
// walks the sequence chunk by chunk, keeping its slice of the float32 state in
// MFMA accumulators for the whole sequence.
//
// Method (chunk of C = 64 tokens, 16-token sub-tiles R = 0..3; log-decays in
// base-2 units, gamma = clamp(g) * log2(e), e = 2^gamma per token and channel):
//   L_r    inclusive cumulative gamma inside r's sub-tile;  tau_R its total
//   ref_R  sum of tau over earlier sub-tiles (chunk-relative start of R)
//   A[r,i] = beta_r sum_c k_rc k_ic 2^(G_rc - G_ic)     i < r   (G = ref + L)
//   P[r,i] =        sum_c q_rc k_ic 2^(G_rc - G_ic)     i <= r
//   U      = (I + A)^-1 Diag(beta) (V - Kc S)     (UT form; Kc = k 2^G, S = state
//            entering the chunk), by block forward substitution over the sub-tiles
//            with the diagonal blocks D_R = (I + A_RR)^-1
//   O      = Qc S + P U                   (Qc = q 2^G)
//   S'     = Diag(2^G_end) S + (k 2^(G_end - G))^T U
// Every 2^(...) above is a product of the per-token factors e (a prefix or suffix
// product inside a token range, times range and sub-tile totals), so the only
// transcendental per element is the one that forms e.
// A and P are built per 16x16 tile pair (R, I <= R) as one dense MFMA product
// of a row operand x 2^(L_r) (<= 1) and a column operand x 2^(ref_R - G_i).
// On off-diagonal tiles the column factor is <= 1; on the diagonal tiles it is
// 2^(-L_i) <= 2^(16 * 5 * log2 e) = e^80 ~ 5.5e34, inside bfloat16's range, so
// diagonal tiles are the same dense product as the others followed by a
// triangular mask - the consequence of the -5 log-decay floor that the orkas.ai
// blog "Kimi K3 architecture" draws in "A lower bound that deleted a GPU code
// path".  The chunk-parallel rewrite itself is the one the Towards-AI article's
// "Kimi Delta Attention (KDA)" section refers to.
//
// Precision (bfloat16 inputs): MFMA operands are bfloat16 with float32
// accumulation.  The output path through the diagonal P tiles (q 2^L and the
// column operand on those tiles, P itself) and U are carried as hi + lo bfloat16
// pairs (three products per pair of split operands); A, Kc, Qc, S and the
// state-update key operand are single bfloat16; the inverses and the block
// substitution run in float32.  float32 inputs use the float32 MFMA throughout.
//
// Schedule of one chunk (eight waves, two per SIMD; "|" = barrier):
//   range decay products (one thread per channel pair and token range) |
//   operands | A and P tile pairs, the diagonal pairs' waves then invert
//   I + A_RR on MFMA from registers | deferred operands (Kc, Qc, transposed
//   state-update keys) | per row tile: Kc S, Qc S, Z = beta (V - Kc S) | block
//   substitution for U (four waves), P to hi / lo rows (four waves) | P U,
//   output tile, state update | output stores, next chunk's inputs to shared
//   memory.
//
// The walk itself is in kda_prefill_body.inc, one text used twice: inside the
// ordinary kernel (chunk_fwd_kernel) and inside a device function (chunk_body)
// that the segmented path's summary kernel calls for its two kinds of workgroup.
// Its summary variant (SUM) drops the query, P-tile and output work, which frees
// the shared memory for all 128 value columns in one workgroup.

#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <bool BF16>
struct Mfma;
template <>
struct Mfma<true> {
  static constexpr int KSTEP = 32, KPL = 8;
  typedef bf16x8 frag;
  typedef __bf16 op_t;
  __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ frag ld(const op_t* p) {
    return *reinterpret_cast<const bf16x8*>(p);
  }
};
template <>
struct Mfma<false> {
  static constexpr int KSTEP = 4, KPL = 1;
  typedef float frag;
  typedef float op_t;
  __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ frag ld(const op_t* p) { return *p; }
};

__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Z = X Y for 16x16 float32 matrices held in the MFMA result layout (lane l
// holds rows 4*(l>>4)+m, column l&15).  X is passed transposed (Xt), Y as is:
// in that form both are already the operands of the k-steps, no data movement.
__device__ __forceinline__ f32x4 mm16(const f32x4& Xt, const f32x4& Y, f32x4 acc) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) acc = mma_f32(Xt[kb], Y[kb], acc);
  return acc;
}

constexpr int kC = 64;    // chunk
constexpr int kSub = 16;  // sub-tile
constexpr int kNSub = 4;

// SUM: the summary-only variant (no query, P or output buffers).
template <typename TIn, int DK, int DVS, bool SUM = false>
struct PrefillLayout {
  static constexpr bool BF16 = sizeof(TIn) == 2;
  typedef typename Mfma<BF16>::op_t op_t;
  static constexpr int OPB = sizeof(op_t);
  static constexpr int PAD = 16 / OPB;
  // [x][DK] operand arrays: rows padded by 32 bytes (288-byte rows at d = 128).  Rows of
  // 272 bytes (16 bytes of padding) measured 3.5% slower over the whole kernel; the other
  // row strides below were swept the same way and are at their best within the budget.
  static constexpr int LDK = DK + 2 * PAD;
  static constexpr int LDC = kC + PAD;  // [x][64] operand arrays (k = token)
  static constexpr int LDF = DK + 4;    // [64][DK] float32
  static constexpr int LDA = kC + 4;    // [64][64] float32

  static constexpr int SZ_K = kC * LDK * OPB;
  static constexpr int SZ_Q = SUM ? 0 : SZ_K;  // raw q
  static constexpr int SZ_Q2 = (BF16 && !SUM) ? kC * LDK * OPB : 0;
  // 2^gamma (float32) for the decay products; then the column operand k 2^-L, as float32
  // (float32 inputs) or as a hi + lo pair of bfloat16 arrays
  static constexpr int SZ_L = (BF16 && 2 * kC * LDK * OPB > kC * LDF * 4) ? 2 * kC * LDK * OPB
                                                                         : kC * LDF * 4;
  static constexpr int SZ_KBT = DK * LDC * OPB;
  static constexpr int SZ_KC = kC * LDK * OPB;
  static constexpr int SZ_QC = SUM ? 0 : SZ_KC;
  // Z^T (float32, [value column][token]) and then, in the same rows, U^T: hi part at
  // element 0, lo part at element ULO (bfloat16); row stride LDZ floats (304 bytes:
  // 16-byte aligned rows, no bank conflicts across 16 rows)
  static constexpr int LDZ = kC + 12;
  static constexpr int LDU = LDZ * 4 / OPB;  // the same rows in operand elements
  static constexpr int ULO = LDC;
  static_assert(!BF16 || ULO + kC <= LDU, "U^T hi and lo share a row");
  static constexpr int SZ_ZU = DVS * LDZ * 4;
  static constexpr int LDD = 16 + 4;  // diagonal blocks of (I + A)^-1, float32 [64][LDD]
  static constexpr int SZ_D = kC * LDD * 4;
  static constexpr int PH1 = SZ_K + SZ_Q + SZ_Q2 + SZ_L;
  static constexpr int PH2 = SZ_KC + SZ_QC + SZ_KBT + SZ_ZU + SZ_D;
  static constexpr int REGION = PH1 > PH2 ? PH1 : PH2;
  // phase-1 view of the shared region: raw inputs, then the A/P operands
  static constexpr int O_K = 0, O_Q = SZ_K, O_Q2 = SZ_K + SZ_Q, O_L = SZ_K + SZ_Q + SZ_Q2;
  // phase-2 view: the state-pass operands
  static constexpr int O_KC = 0, O_QC = SZ_KC, O_KBT = SZ_KC + SZ_QC, O_ZU = O_KBT + SZ_KBT;
  static constexpr int O_D = O_ZU + SZ_ZU;
  // buffers outside the region
  static constexpr int SZ_AW = kC * LDA * 4;  // A (float32), then the output staging
  static constexpr int SZ_P = SUM ? 0 : kC * LDA * 4;
  static constexpr int O_A = REGION;
  static constexpr int O_P = O_A + SZ_AW;
  static constexpr int LDV = DVS + PAD;  // v slice, token-major [64][LDV]
  static constexpr int O_V = O_P + SZ_P;
  static constexpr int O_ST = O_V + kC * LDV * OPB;
  static constexpr int O_SM = O_ST + DVS * LDK * OPB;
  // small float32 arrays: beta[64], range totals [NRNG][DK], pair[6][DK], egam[DK]
  // (the scan runs one thread per channel pair and range of a 512-thread group)
  static constexpr int NRNG = 2 * 512 / DK;
  static constexpr int SM_BETA = 0, SM_RNG = 64, SM_PAIR = 64 + NRNG * DK;
  static constexpr int SM_EGAM = SM_PAIR + 6 * DK;
  static constexpr int SZ_SM = (SM_EGAM + DK) * 4;
  static constexpr int TOTAL = O_SM + SZ_SM;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// The walk of one workgroup, as a device function for the split summary pass.
// SUM: a summary-pass workgroup that needs no query, P tiles or outputs (the
// zero-start state or the transition of a segment after the first), carrying all
// of its DVS columns.
// SPLIT: a part of the split summary pass, whose segment range and transition
// workgroups come from seg_first, seg_count and with_p.
template <typename TIn, typename TOut, int DK, int DV, int DVS, bool GATE, bool SUM, bool SPLIT>
__device__ __forceinline__ void chunk_body(const PrefillArgs& p, const int64_t block_index) {
#include "kda_prefill_body.inc"
}

template <typename TIn, typename TOut, int DK, int DV, int DVS, bool GATE>
__global__ void __launch_bounds__(512) chunk_fwd_kernel(PrefillArgs p) {
  constexpr bool SUM = false, SPLIT = false;
  const int64_t block_index = blockIdx.x;
#include "kda_prefill_body.inc"
}

// The split summary pass (bfloat16, d_k = d_v = 128): workgroups [0, split) walk
// segment 0 as the ordinary kernel does (a0), the rest are summary workgroups of
// 128 columns for the later segments (a1).  split is a multiple of 8, so both parts
// keep the ordinary mapping of a unit's workgroups onto one XCD.
template <typename TOut, bool GATE>
__global__ void __launch_bounds__(512) chunk_fwd_summary_kernel(PrefillArgs a0, PrefillArgs a1,
                                                                int64_t split) {
  const int64_t x = blockIdx.x;
  if (x < split)
    chunk_body<__bf16, TOut, 128, 128, 64, GATE, false, true>(a0, x);
  else
    chunk_body<__bf16, TOut, 128, 128, 128, false, true, true>(a1, x - split);
}

// Units (b, segment, h) and workgroups per unit of one launch.
template <int DK, int DV, int DVS>
int64_t launch_units(const PrefillArgs& a, int* slices) {
  constexpr int NSLICE = DV / DVS, NPSL = DK / DVS;
  *slices = (a.mode && a.with_p) ? NSLICE + NPSL : NSLICE;
  return a.B * (a.seg_count > 0 ? a.seg_count : (a.nseg > 1 ? a.nseg - 1 : 1)) * a.H;
}

template <typename TIn, typename TOut, int DK, int DV, int DVS>
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  typedef PrefillLayout<TIn, DK, DVS> Lay;
  auto kern = a.ogate ? chunk_fwd_kernel<TIn, TOut, DK, DV, DVS, true>
                      : chunk_fwd_kernel<TIn, TOut, DK, DV, DVS, false>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     Lay::TOTAL);
  if (e != hipSuccess) return e;
  int slices = 0;
  const int64_t units = launch_units<DK, DV, DVS>(a, &slices);
  const int64_t grid = prefill_grid(units, slices);
  kern<<<dim3((unsigned)grid), dim3(512), Lay::TOTAL, stream>>>(a);
  return hipGetLastError();
}

bool summary_split_ok(int dk, int dv, bool in_bf16, int chunk) {
  return in_bf16 && dk == 128 && dv == 128 && chunk == 64;
}

template <typename TOut>
hipError_t launch_summary(const PrefillArgs& a0, const PrefillArgs& a1, hipStream_t stream) {
  constexpr int L0 = PrefillLayout<__bf16, 128, 64>::TOTAL;
  constexpr int L1 = PrefillLayout<__bf16, 128, 128, true>::TOTAL;
  constexpr int LDS = L0 > L1 ? L0 : L1;
  static_assert(LDS <= 160 * 1024, "LDS budget");
  auto kern = a0.ogate ? chunk_fwd_summary_kernel<TOut, true> : chunk_fwd_summary_kernel<TOut, false>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
  if (e != hipSuccess) return e;
  int s0 = 0, s1 = 0;
  const int64_t u0 = launch_units<128, 128, 64>(a0, &s0);
  const int64_t u1 = launch_units<128, 128, 128>(a1, &s1);
  const int64_t split = prefill_grid(u0, s0);
  const int64_t grid = split + prefill_grid(u1, s1);
  kern<<<dim3((unsigned)grid), dim3(512), LDS, stream>>>(a0, a1, split);
  return hipGetLastError();
}

hipError_t chunk_fwd_summary(const PrefillArgs& a0, const PrefillArgs& a1, bool out_bf16,
                             hipStream_t s) {
  return out_bf16 ? launch_summary<__bf16>(a0, a1, s) : launch_summary<float>(a0, a1, s);
}

// d_v slice width per workgroup (must match the instantiations in chunk_fwd).
int prefill_slice(int dk, int dv, bool in_bf16) {
  (void)dv;
  if (!in_bf16) return 64;
  return dk == 128 ? 64 : 32;
}

int64_t prefill_grid(int64_t units, int slices) { return ((units + 7) / 8) * 8 * slices; }

hipError_t chunk_fwd(const PrefillArgs& a, int dk, int dv, bool in_bf16, bool out_bf16,
                     hipStream_t s) {
  if (in_bf16) {
    if (out_bf16) {
      if (dk == 128 && dv == 128) return launch_prefill<__bf16, __bf16, 128, 128, 64>(a, s);
      if (dk == 128 && dv == 64) return launch_prefill<__bf16, __bf16, 128, 64, 64>(a, s);
      if (dk == 64 && dv == 128) return launch_prefill<__bf16, __bf16, 64, 128, 32>(a, s);
      return launch_prefill<__bf16, __bf16, 64, 64, 32>(a, s);
    }
    if (dk == 128 && dv == 128) return launch_prefill<__bf16, float, 128, 128, 64>(a, s);
    if (dk == 128 && dv == 64) return launch_prefill<__bf16, float, 128, 64, 64>(a, s);
    if (dk == 64 && dv == 128) return launch_prefill<__bf16, float, 64, 128, 32>(a, s);
    return launch_prefill<__bf16, float, 64, 64, 32>(a, s);
  }
  if (out_bf16) return launch_prefill<float, __bf16, 64, 64, 64>(a, s);
  return launch_prefill<float, float, 64, 64, 64>(a, s);
}

}  // namespace kda
