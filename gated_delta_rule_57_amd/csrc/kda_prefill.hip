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

template <typename TIn, int DK, int DVS>
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
  static constexpr int SZ_Q2 = BF16 ? kC * LDK * OPB : 0;
  // 2^gamma (float32) for the decay products; then the column operand k 2^-L, as float32
  // (float32 inputs) or as a hi + lo pair of bfloat16 arrays
  static constexpr int SZ_L = (BF16 && 2 * kC * LDK * OPB > kC * LDF * 4) ? 2 * kC * LDK * OPB
                                                                         : kC * LDF * 4;
  static constexpr int SZ_KBT = DK * LDC * OPB;
  static constexpr int SZ_QC = kC * LDK * OPB;
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
  static constexpr int PH1 = 2 * SZ_K + SZ_Q2 + SZ_L;
  static constexpr int PH2 = 2 * SZ_QC + SZ_KBT + SZ_ZU + SZ_D;
  static constexpr int REGION = PH1 > PH2 ? PH1 : PH2;
  // phase-1 view of the shared region: raw inputs, then the A/P operands
  static constexpr int O_K = 0, O_Q = SZ_K, O_Q2 = 2 * SZ_K, O_L = 2 * SZ_K + SZ_Q2;
  // phase-2 view: the state-pass operands
  static constexpr int O_KC = 0, O_QC = SZ_QC, O_KBT = 2 * SZ_QC, O_ZU = O_KBT + SZ_KBT;
  static constexpr int O_D = O_ZU + SZ_ZU;
  // buffers outside the region
  static constexpr int SZ_AW = kC * LDA * 4;  // A (float32), then the output staging
  static constexpr int O_A = REGION;
  static constexpr int O_P = O_A + SZ_AW;
  static constexpr int LDV = DVS + PAD;  // v slice, token-major [64][LDV]
  static constexpr int O_V = O_P + kC * LDA * 4;
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

template <typename TIn, typename TOut, int DK, int DV, int DVS, bool GATE>
__global__ void __launch_bounds__(512) chunk_fwd_kernel(PrefillArgs p) {
  typedef PrefillLayout<TIn, DK, DVS> Lay;
  constexpr bool BF16 = Lay::BF16;
  typedef Mfma<BF16> M;
  typedef typename M::op_t op_t;
  typedef typename M::frag frag;
  constexpr int NW = 8, NT = 512;
  constexpr int KS = M::KSTEP, KPL = M::KPL;
  constexpr int LDK = Lay::LDK, LDC = Lay::LDC, LDF = Lay::LDF, LDA = Lay::LDA;
  constexpr int NSLICE = DV / DVS;
  constexpr int NJT = DVS / 16;          // value-column tiles
  constexpr int NJW = NJT / 2;           // value-column tiles per wave (two waves per row tile)
  constexpr int NST = (DK / 16) * NJT;   // state tiles
  constexpr int SPW = NST / NW;          // state tiles per wave
  // channel-major phases: one thread per (channel pair, range of RL tokens)
  constexpr int NCP = DK / 2;            // channel pairs
  constexpr int NR = NT / NCP;           // token ranges
  constexpr int RL = kC / NR;            // tokens per range
  constexpr int RPS = kSub / RL;         // ranges per sub-tile
  static_assert(NR == Lay::NRNG && NR * NCP == NT && RL * NR == kC && RPS * RL == kSub, "ranges");
  constexpr int E16 = 16 / sizeof(TIn);  // input elements per 16-byte load
  constexpr int NPF = kC * DK / E16 / NT;
  constexpr int PPV = DVS / E16;         // 16-byte pieces per token of the v slice
  constexpr int NPV = (kC * PPV + NT - 1) / NT;  // v pieces per thread (rounded up)
  static_assert(NPF * E16 * NT == kC * DK && PPV * E16 == DVS, "load layout");
  static_assert(SPW * NW == NST && NJW >= 1, "layout");

  extern __shared__ __align__(16) unsigned char smem[];
  op_t* sK = reinterpret_cast<op_t*>(smem + Lay::O_K);
  op_t* sQ = reinterpret_cast<op_t*>(smem + Lay::O_Q);
  op_t* sQ2 = reinterpret_cast<op_t*>(smem + Lay::O_Q2);
  float* sL = reinterpret_cast<float*>(smem + Lay::O_L);
  op_t* sKdH = reinterpret_cast<op_t*>(smem + Lay::O_L);  // k 2^-L, hi part (bfloat16 inputs)
  op_t* sKdL = sKdH + kC * LDK;                            // lo part
  op_t* sKc = reinterpret_cast<op_t*>(smem + Lay::O_KC);
  op_t* sQc = reinterpret_cast<op_t*>(smem + Lay::O_QC);
  op_t* sKbT = reinterpret_cast<op_t*>(smem + Lay::O_KBT);
  float* sZT = reinterpret_cast<float*>(smem + Lay::O_ZU);
  op_t* sUT = reinterpret_cast<op_t*>(smem + Lay::O_ZU);
  op_t* sUT2 = sUT + Lay::ULO;  // lo part (bf16 only)
  float* sD = reinterpret_cast<float*>(smem + Lay::O_D);
  constexpr int LDZ = Lay::LDZ, LDU = Lay::LDU, LDD = Lay::LDD;
  float* sA = reinterpret_cast<float*>(smem + Lay::O_A);
  float* sP = reinterpret_cast<float*>(smem + Lay::O_P);
  op_t* sV = reinterpret_cast<op_t*>(smem + Lay::O_V);
  constexpr int LDV = Lay::LDV;
  op_t* sST = reinterpret_cast<op_t*>(smem + Lay::O_ST);
  float* sm = reinterpret_cast<float*>(smem + Lay::O_SM);
  float* sBeta = sm + Lay::SM_BETA;
  float* sRng = sm + Lay::SM_RNG;
  float* sPair = sm + Lay::SM_PAIR;
  float* sEGam = sm + Lay::SM_EGAM;

  // Lane indices are refreshed at the top of every chunk (see refresh_lane):
  // the many per-lane shared-memory addresses derived from them are then cheap
  // to recompute inside the loop instead of occupying registers across it.
  int tid = threadIdx.x, lane, l16, lg, kofs;
  auto refresh_lane = [&]() {
    asm volatile("" : "+v"(tid));
    lane = tid & 63;
    l16 = lane & 15;
    lg = lane >> 4;
    kofs = lg * KPL;
  };
  refresh_lane();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rt = wave & 3;            // row tile of the chunk owned by this wave
  const int jt0 = (wave >> 2) * NJW;  // its first value-column tile

  // Workgroup -> (unit, slice), unit = (b, segment, h): consecutive workgroups
  // are dealt round-robin to the 8 XCDs, so give all slices of a unit the same
  // XCD (and L2).  With several segments each launch covers all but one: the
  // summary pass (mode 1) every segment but the last, with DK / DVS more slices
  // that carry the segment's transition matrix; the output pass (mode 0) every
  // segment but the first, whose outputs the summary pass already wrote (its
  // workgroups start from the true initial state).
  constexpr int NPSL = DK / DVS;
  const int nsl = p.mode ? NSLICE + NPSL : NSLICE;
  const int64_t nsg = p.nseg > 1 ? p.nseg - 1 : 1;
  const int64_t seg0 = (p.mode == 0 && p.nseg > 1) ? 1 : 0;  // first segment covered
  const int64_t x = blockIdx.x;
  const int64_t grp = x / (8 * nsl);
  const int gi = (int)(x % (8 * nsl));
  const int64_t unit = grp * 8 + (gi % 8);
  const int slice = gi / 8;
  if (unit >= p.B * nsg * p.H) return;
  const int64_t h = unit % p.H, bj = unit / p.H, seg = bj % nsg + seg0, b = bj / nsg;
  const bool pmode = slice >= NSLICE;  // transition workgroup (mode 1 only)
  if (pmode && seg == 0) return;       // segment 0's transition is never used
  const int j0 = (pmode ? slice - NSLICE : slice) * DVS;
  const int64_t T = p.T, H = p.H;
  const RangeCheck rc{p.range_flags};  // checks only in a KDA_DEBUG_RANGE build
  const int64_t tb = seg * p.seg_len;                             // first token
  const int64_t te = (T - tb) < p.seg_len ? T : tb + p.seg_len;   // one past the last
  // outputs (o, checkpoints, the final state) come from the output pass and, for
  // segment 0, from the summary pass's workgroups that walk it from the initial state
  const bool emit = p.mode == 0 || (seg == 0 && !pmode);

  const TIn* gq = reinterpret_cast<const TIn*>(p.q);
  const TIn* gk = reinterpret_cast<const TIn*>(p.k);
  const TIn* gv = reinterpret_cast<const TIn*>(p.v);
  const TIn* gg = reinterpret_cast<const TIn*>(p.g);
  const TIn* gb = reinterpret_cast<const TIn*>(p.beta);
  TOut* go = reinterpret_cast<TOut*>(p.o);
  const int64_t head_off = (b * H + h) * (int64_t)DK * DV;       // [B, H, DK, DV] states
  const int64_t seg_unit = (b * p.nseg + seg) * H + h;           // [B, nseg, H, ...] states

  // ---- state slice in accumulators: a wave holds one value-column tile jt = wave % NJT
  // and SPW key-channel tiles ct = (wave / NJT) SPW + i
  const float* src = nullptr;  // entry state (row stride DV), NULL = zeros
  if (seg > 0) {  // output pass: the scanned entry state; summary pass: zeros (or identity)
    if (p.mode == 0) src = p.seg_in + seg_unit * DK * DV;
  } else if (p.s0) {
    src = p.s0 + head_off;
  }
  f32x4 Sacc[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int ct = (wave / NJT) * SPW + i, jt = wave % NJT;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int c = 16 * ct + 4 * lg + m, jv = 16 * jt + l16;
      if (pmode)
        Sacc[i][m] = (c == j0 + jv) ? 1.f : 0.f;  // identity columns j0..j0+DVS-1
      else
        Sacc[i][m] = src ? src[(int64_t)c * DV + j0 + jv] : 0.f;
    }
  }
  auto store_state_operand = [&]() {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int ct = (wave / NJT) * SPW + i, jt = wave % NJT;
      op_t* dst = sST + (16 * jt + l16) * LDK + 16 * ct + 4 * lg;
#pragma unroll
      for (int m = 0; m < 4; ++m) dst[m] = from_f32<op_t>(Sacc[i][m]);
    }
  };
  store_state_operand();

  // ---- register prefetch of one chunk of raw inputs (16-byte pieces).  Addresses
  // are a uniform 64-bit chunk base plus 32-bit per-thread offsets.
  float4 pk[NPF], pq[NPF], pg[NPF];
  float4 pv[NPV];  // stays zero for transition workgroups
#pragma unroll
  for (int i = 0; i < NPV; ++i) pv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  TIn pbeta = from_f32<TIn>(0.f);  // kept raw: converting here would wait for the load
  // output gate of the current chunk: one unit of 8 consecutive values of a row of the
  // slice per thread (units 0 .. 64 DVS / 8 - 1), raw, loaded at the top of the chunk
  constexpr int GU = DVS / 8;                 // gate units per row
  constexpr int GPC = 8 * sizeof(TIn) / 16;   // 16-byte pieces per unit
  static_assert(kC * GU <= NT, "one gate unit per thread");
  float4 pz[GPC];
#pragma unroll
  for (int i = 0; i < GPC; ++i) pz[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  // token strides (elements); offsets inside one chunk fit in 32 bits
  const uint32_t rs_k = (uint32_t)(H * DK), rs_v = (uint32_t)(H * DV), rs_b = (uint32_t)H;
  // Rows past the end of the sequence load the last valid token (always in
  // bounds) and are zeroed when staged, so the loads themselves are branch-free.
  // The loads are issued in four parts spread over the chunk's phases, so that
  // the memory pipeline is not asked for a whole chunk at once: v at the top of
  // the chunk, k after the decay products, q before the row-tile products, g and
  // beta before the substitution (placements swept; these measured fastest).
  auto prefetch = [&](int64_t t0, int part) {
    const int64_t cb = (b * T + t0) * H + h;
    const int last = (int)((te - t0) < kC ? (te - t0) : kC) - 1;
    if (part == 0) {
      const TIn* vb = gv + cb * DV + j0;
      if (!pmode) {
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
          const int pc = tid + NT * i;
          const int r = min(pc / PPV, last), c = (pc % PPV) * E16;
          if (pc < kC * PPV)
            pv[i] = ld_at<float4>(vb, ((uint32_t)r * rs_v + (uint32_t)c) * (uint32_t)sizeof(TIn));
        }
      }
      return;
    }
    const TIn* base = (part == 1 ? gk : part == 2 ? gq : gg) + cb * DK;
#pragma unroll
    for (int i = 0; i < NPF; ++i) {
      const int pc = tid + NT * i;
      const int r = min(pc / (DK / E16), last), c = (pc % (DK / E16)) * E16;
      const float4 x = ld_at<float4>(base, ((uint32_t)r * rs_k + (uint32_t)c) * (uint32_t)sizeof(TIn));
      if (part == 1) pk[i] = x;
      else if (part == 2) pq[i] = x;
      else pg[i] = x;
    }
    if (part == 3 && tid < kC)
      pbeta = ld_at<TIn>(gb + cb, (uint32_t)min(tid, last) * rs_b * (uint32_t)sizeof(TIn));
  };
  // Prefetched chunk starting at token t0 -> shared memory: k, q raw; g -> 2^gamma
  // (float32); v; beta.  Rows past the end become beta = 0, g = 0, k = q = v = 0
  // tokens, which leave the state unchanged.
  auto stage = [&](int64_t t0) {
    const int nvalid = (int)((te - t0) < kC ? (te - t0) : kC);
#pragma unroll
    for (int i = 0; i < NPF; ++i) {
      const int pc = tid + NT * i;
      const int r = pc / (DK / E16), c = (pc % (DK / E16)) * E16;
      // bitwise masks (a select between registers here becomes a select between
      // addresses, which sends the prefetch registers to scratch memory)
      const uint32_t mk = r < nvalid ? 0xffffffffu : 0u;
      *reinterpret_cast<uint4*>(sK + r * LDK + c) = mask4(pk[i], mk);
      *reinterpret_cast<uint4*>(sQ + r * LDK + c) = mask4(pq[i], mk);
      float gf[E16];
      unpack16(pg[i], (TIn*)nullptr, gf);
      // per-token decay 2^gamma (1 on padded rows)
      if (p.gate_logits) {  // raw decay logits: negative softplus, then the floor
#pragma unroll
        for (int e = 0; e < E16; ++e) gf[e] = exp2_hw(gamma_from_logit(gf[e]));
      } else {
#pragma unroll
        for (int e = 0; e < E16; ++e) gf[e] = exp2_hw(clamp_log_decay(gf[e]) * kLog2e);
      }
#pragma unroll
      for (int e = 0; e < E16; ++e)
        gf[e] = __uint_as_float((__float_as_uint(gf[e]) & mk) | (0x3f800000u & ~mk));
      if constexpr (E16 == 8) {
        store8(sL + r * LDF + c, gf);
      } else {
        *reinterpret_cast<f32x4*>(sL + r * LDF + c) = f32x4{gf[0], gf[1], gf[2], gf[3]};
      }
    }
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const int pc = tid + NT * i;
      const int r = pc / PPV, c = (pc % PPV) * E16;
      if (pc < kC * PPV)
        *reinterpret_cast<uint4*>(sV + r * LDV + c) = mask4(pv[i], r < nvalid ? 0xffffffffu : 0u);
    }
    if (tid < kC) sBeta[tid] = (tid < nvalid) ? to_f32(pbeta) : 0.f;
  };

  const int64_t nchunks = (te - tb + kC - 1) / kC;
  // listed checkpoint positions: the first one past this walk's first chunk
  int64_t ck_next = 0;
  if (emit && p.ck && p.ck_pos) {
    int64_t lo = 0, hi = p.n_ck;
    while (lo < hi) {
      const int64_t mid = (lo + hi) / 2;
      if (p.ck_pos[mid] < tb + kC) lo = mid + 1;
      else hi = mid;
    }
    ck_next = lo;
  }
  for (int part = 0; part < 4; ++part) prefetch(tb, part);
  stage(tb);
  __syncthreads();

  for (int64_t n = 0; n < nchunks; ++n) {
    const int64_t t0 = tb + n * kC;
    refresh_lane();
    // Next chunk's inputs: loaded while this chunk computes, staged at its end.  The
    // last chunk reloads itself (in bounds, never used) so that loads and staging
    // are unconditional.
    const int64_t tn = (n + 1 < nchunks) ? t0 + kC : t0;
    prefetch(tn, 0);
    if constexpr (GATE) {
      if (emit && tid < kC * GU) {
        const int r = min(tid / GU, (int)((te - t0) < kC ? (te - t0) : kC) - 1);
        const int c = (tid % GU) * 8;
        const TIn* zb = reinterpret_cast<const TIn*>(p.ogate) + ((b * T + t0) * H + h) * DV + j0;
#pragma unroll
        for (int i = 0; i < GPC; ++i)
          pz[i] = ld_at<float4>(zb, ((uint32_t)r * rs_v + (uint32_t)c) * (uint32_t)sizeof(TIn) +
                                        16u * (uint32_t)i);
      }
    }
    // ---- decay products: one thread per (channel pair, token range); the ranges'
    // products go to shared memory for the sub-tile offsets
    const int cp = tid % NCP, hr = tid / NCP, c0 = 2 * cp, r0 = RL * hr;
    f32x2 Lr[RL];  // 2^gamma of both channels, per token of this range
    {
#pragma unroll
      for (int j = 0; j < RL; ++j)
        Lr[j] = *reinterpret_cast<const f32x2*>(sL + (r0 + j) * LDF + c0);
      f32x2 acc = Lr[0];
#pragma unroll
      for (int j = 1; j < RL; ++j) acc *= Lr[j];
      *reinterpret_cast<f32x2*>(sRng + hr * DK + c0) = acc;
    }
    __syncthreads();

    prefetch(tn, 1);
    // ---- operands (same thread, same elements, so the updates are in place); two
    // channels at a time: packed conversions, 32-bit shared-memory accesses
    typedef typename std::conditional<BF16, uint32_t, f32x2>::type op2_t;
    auto ld2 = [](const op_t* p) { return *reinterpret_cast<const op2_t*>(p); };
    auto st2 = [](op_t* p, op2_t x) { *reinterpret_cast<op2_t*>(p) = x; };
    op2_t dKc[RL], dQc[RL], dKb[RL];
    {
      const int R = hr / RPS, part = hr % RPS;
      // decay products (2^ of the log-decay sums): tau[J] over sub-tile J, off over the
      // earlier ranges of this thread's sub-tile, own over its own range
      f32x2 tau[kNSub], off = {1.f, 1.f};
#pragma unroll
      for (int J = 0; J < kNSub; ++J) {
        tau[J] = *reinterpret_cast<const f32x2*>(sRng + (J * RPS) * DK + c0);
#pragma unroll
        for (int u = 1; u < RPS; ++u)
          tau[J] *= *reinterpret_cast<const f32x2*>(sRng + (J * RPS + u) * DK + c0);
      }
#pragma unroll
      for (int u = 0; u + 1 < RPS; ++u) {  // earlier ranges of this sub-tile
        const f32x2 t = *reinterpret_cast<const f32x2*>(sRng + (R * RPS + u) * DK + c0);
        if (u < part) off *= t;
      }
      const f32x2 own = *reinterpret_cast<const f32x2*>(sRng + hr * DK + c0);
      if (hr == 0) {
        const f32x2 t01 = tau[0] * tau[1], t12 = tau[1] * tau[2];
        *reinterpret_cast<f32x2*>(sPair + 0 * DK + c0) = tau[0];          // (1,0)
        *reinterpret_cast<f32x2*>(sPair + 1 * DK + c0) = t01;             // (2,0)
        *reinterpret_cast<f32x2*>(sPair + 2 * DK + c0) = tau[1];          // (2,1)
        *reinterpret_cast<f32x2*>(sPair + 3 * DK + c0) = t01 * tau[2];    // (3,0)
        *reinterpret_cast<f32x2*>(sPair + 4 * DK + c0) = t12;             // (3,1)
        *reinterpret_cast<f32x2*>(sPair + 5 * DK + c0) = tau[2];          // (3,2)
        *reinterpret_cast<f32x2*>(sEGam + c0) = t01 * (tau[2] * tau[3]);
      }
      f32x2 eref = {1.f, 1.f}, ebar = {1.f, 1.f};  // 2^ref, 2^suf
#pragma unroll
      for (int J = 0; J < kNSub; ++J) {
        if (J < R) eref *= tau[J];
        else ebar *= tau[J];
      }
      // 2^L_j (L = inclusive sub-tile sum) and 2^-L_j as prefix / suffix products of
      // 2^gamma over the range, started from the range's offset inside its sub-tile
      f32x2 ep[RL], em[RL];
      {
        const f32x2* f = Lr;
        // 2^-L at the range's last token: the reciprocal (to 1 ulp) of its prefix
        // product; a sub-tile's product stays >= 2^(-16 * 5 log2 e), a normal float
        const f32x2 po = off * own;
        f32x2 pre = off, sp = f32x2{__builtin_amdgcn_rcpf(po.x), __builtin_amdgcn_rcpf(po.y)};
#pragma unroll
        for (int j = 0; j < RL; ++j) {
          pre *= f[j];
          ep[j] = pre;
        }
#pragma unroll
        for (int j = RL - 1; j >= 0; --j) {
          em[j] = sp;
          sp *= f[j];
        }
      }
#pragma unroll
      for (int j = 0; j < RL; ++j) {
        const int r = r0 + j;
        const f32x2 kf = unpack2(ld2(sK + r * LDK + c0)), qf = unpack2(ld2(sQ + r * LDK + c0));
        const f32x2 kr = kf * ep[j], qr = qf * ep[j], kd = kf * em[j];
        {
          constexpr float lim = BF16 ? kBf16Max : 3.4028235e38f;
          rc.factors(ep[j].x, em[j].x);
          rc.factors(ep[j].y, em[j].y);
          rc.operand(kr.x, lim), rc.operand(kr.y, lim), rc.operand(qr.x, lim);
          rc.operand(qr.y, lim), rc.operand(kd.x, lim), rc.operand(kd.y, lim);
        }
        st2(sK + r * LDK + c0, pack2(kr, (op2_t*)nullptr));
        const op2_t qh = pack2(qr, (op2_t*)nullptr);
        st2(sQ + r * LDK + c0, qh);
        if constexpr (BF16) {
          st2(sQ2 + r * LDK + c0, pack2(qr - unpack2(qh), (op2_t*)nullptr));
          const op2_t kh = pack2(kd, (op2_t*)nullptr);
          st2(sKdH + r * LDK + c0, kh);
          st2(sKdL + r * LDK + c0, pack2(kd - unpack2(kh), (op2_t*)nullptr));
        } else {
          *reinterpret_cast<f32x2*>(sL + r * LDF + c0) = kd;
        }
        dKc[j] = pack2(kr * eref, (op2_t*)nullptr);
        dQc[j] = pack2(qr * eref, (op2_t*)nullptr);
        dKb[j] = pack2(kd * ebar, (op2_t*)nullptr);
      }
    }
    __syncthreads();

    // ---- A and P tiles, every tile pair one dense product.  Waves 0-3 take the six
    // off-diagonal pairs (two, two, one, one); wave 4 + R takes the diagonal pair
    // (R, R) and inverts I + A_RR right away, keeping the inverse in registers (the
    // triangular factor's shared-memory slots alias operands other waves still read).
    f32x4 Dinv = {0.f, 0.f, 0.f, 0.f};
    // DIAG is a compile-time tag, so that each k-step is straight-line code whose
    // shared-memory loads the compiler can issue ahead of the previous step's MFMAs.
    auto tile_pair = [&](auto diag_tag, const int R, const int I) {
      constexpr bool DIAG = decltype(diag_tag)::value;
      const float* pair = sPair + (R * (R - 1) / 2 + I) * DK;  // used off the diagonal only
      f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
      const int row = kSub * R + l16, col = kSub * I + l16;
      // beta of this lane's four result rows, read before the tile's stores (one read)
      const f32x4 brow = *reinterpret_cast<const f32x4*>(sBeta + kSub * R + 4 * lg);
#pragma unroll
      for (int kk = 0; kk < DK; kk += KS) {
        const int k0 = kk + kofs;
        const frag aK = M::ld(sK + row * LDK + k0);
        const frag aQ = M::ld(sQ + row * LDK + k0);
        if constexpr (BF16 && DIAG) {
          // diagonal tile: column operand straight from its hi / lo arrays; P takes
          // the three products of the split pairs
          const frag aQ2 = M::ld(sQ2 + row * LDK + k0);
          const frag bh = M::ld(sKdH + col * LDK + k0), bl = M::ld(sKdL + col * LDK + k0);
          accA = M::mma(aK, bh, accA);
          accP = M::mma(aQ, bh, accP);
          accP = M::mma(aQ2, bh, accP);
          accP = M::mma(aQ, bl, accP);
        } else if constexpr (BF16) {
          // off-diagonal tile: hi part x the pair's decay 2^(ref_R - ref_I) (<= 1),
          // one bfloat16 operand for both products
          const frag raw = M::ld(sKdH + col * LDK + k0);
          float pf[8];
          load8(pair + k0, pf);
          frag b;
#pragma unroll
          for (int e = 0; e < 8; ++e) b[e] = (__bf16)((float)raw[e] * pf[e]);
          accA = M::mma(aK, b, accA);
          accP = M::mma(aQ, b, accP);
        } else {
          float cf = sL[col * LDF + k0];
          if constexpr (!DIAG) cf *= pair[k0];
          accA = M::mma(aK, cf, accA);
          accP = M::mma(aQ, cf, accP);
        }
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = kSub * R + 4 * lg + m, i = col;
        sA[r * LDA + i] = (!DIAG || i < r) ? brow[m] * accA[m] : 0.f;
        sP[r * LDA + i] = (!DIAG || i <= r) ? accP[m] : 0.f;
        rc.finite((!DIAG || i < r) ? accA[m] : 0.f, kRangeTile);
        rc.finite((!DIAG || i <= r) ? accP[m] : 0.f, kRangeTile);
      }
      return DIAG ? accA * brow : accA;  // diagonal: beta-scaled A rows
    };
    if (wave < 4) {
      // (1,0) (3,1) | (2,0) (3,2) | (2,1) | (3,0)
      const int R0 = wave == 0 ? 1 : wave == 1 ? 2 : wave == 2 ? 2 : 3;
      const int I0 = wave == 2 ? 1 : 0;
      tile_pair(std::false_type{}, R0, I0);
      if (wave < 2) tile_pair(std::false_type{}, 3, wave + 1);
    } else {
      const int R = wave - 4;
      const f32x4 acc = tile_pair(std::true_type{}, R, R);
      // Nd: this lane's entries of A_RR (rows 4 lg + m, column l16), as written to
      // sA; Nt: the transposed entries, read back from sA (same wave, in order)
      f32x4 Nd, Nt, Id;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = 4 * lg + m;
        Nd[m] = (l16 < r) ? acc[m] : 0.f;  // acc is already beta-scaled
        Id[m] = (r == l16) ? 1.f : 0.f;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int m = 0; m < 4; ++m) Nt[m] = sA[(kSub * R + l16) * LDA + kSub * R + 4 * lg + m];
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      const f32x4 N2 = mm16(Nt, Nd, z), N2t = mm16(Nd, Nt, z);
      const f32x4 N4 = mm16(N2t, N2, z), N4t = mm16(N2, N2t, z);
      const f32x4 N8 = mm16(N4t, N4, z);
      const f32x4 X1 = Id - Nd, X1t = Id - Nt;
      const f32x4 X2 = mm16(X1t, N2, X1), X2t = mm16(N2, X1t, X1t);
      const f32x4 X3 = mm16(X2t, N4, X2), X3t = mm16(N4, X2t, X2t);
      Dinv = mm16(X3t, N8, X3);  // (I + A_RR)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8)
    }
    // Of the tiles above the diagonal only (0,1) and (2,3) are ever read (by the
    // row-tile products, whose k-steps span 32 tokens); A's are never read.
    if (tid < 128) {
      const int u = tid >> 6, w = tid & 63;
      const int r = 32 * u + (w >> 2), i = 32 * u + kSub + 4 * (w & 3);
      *reinterpret_cast<f32x4*>(sP + r * LDA + i) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();

    // ---- deferred operands into the released region (channel-major threads):
    // k 2^(G_end - G) transposed (token-contiguous: one piece per channel), k 2^G and
    // q 2^G row-major.
    if constexpr (BF16) {
      uint32_t w0[RL / 2], w1[RL / 2];  // bf16 pairs of tokens, channel c0 / c0 + 1
#pragma unroll
      for (int i = 0; i < RL / 2; ++i) {
        w0[i] = (dKb[2 * i] & 0xffffu) | (dKb[2 * i + 1] << 16);
        w1[i] = (dKb[2 * i] >> 16) | (dKb[2 * i + 1] & 0xffff0000u);
      }
      if constexpr (RL == 8) {
        *reinterpret_cast<uint4*>(sKbT + c0 * LDC + r0) = make_uint4(w0[0], w0[1], w0[2], w0[3]);
        *reinterpret_cast<uint4*>(sKbT + (c0 + 1) * LDC + r0) = make_uint4(w1[0], w1[1], w1[2], w1[3]);
      } else {
        static_assert(RL == 4, "range length");
        *reinterpret_cast<uint2*>(sKbT + c0 * LDC + r0) = make_uint2(w0[0], w0[1]);
        *reinterpret_cast<uint2*>(sKbT + (c0 + 1) * LDC + r0) = make_uint2(w1[0], w1[1]);
      }
    } else {
      static_assert(BF16 || RL == 4, "range length");
      *reinterpret_cast<f32x4*>(sKbT + c0 * LDC + r0) = f32x4{dKb[0].x, dKb[1].x, dKb[2].x, dKb[3].x};
      *reinterpret_cast<f32x4*>(sKbT + (c0 + 1) * LDC + r0) =
          f32x4{dKb[0].y, dKb[1].y, dKb[2].y, dKb[3].y};
    }
#pragma unroll
    for (int j = 0; j < RL; ++j) {
      st2(sKc + (r0 + j) * LDK + c0, dKc[j]);
      st2(sQc + (r0 + j) * LDK + c0, dQc[j]);
    }
    // ---- diagonal blocks D_R = (I + A_RR)^-1, computed with the A tiles, to shared
    // memory (float32) for the substitution below
    if (wave >= 4) {
      const int R = wave - 4;
#pragma unroll
      for (int m = 0; m < 4; ++m) sD[(kSub * R + 4 * lg + m) * LDD + l16] = Dinv[m];
    }
    __syncthreads();

    prefetch(tn, 2);
    // ---- per row tile, over the key channels: Y = Kc S and Qc S; Z = V - Y, stored
    // transposed and times beta (float32) for the substitution
    constexpr int NKT = kC / KS;  // k-steps over the chunk's tokens
    const int kend = 16 * rt + 16;  // P rows of this tile vanish beyond kend
    f32x4 Oacc[NJW];
    // output staging [64][LDO]: in the output dtype, or in float32 when the gate is
    // applied at the store (one rounding, after the gate)
    typedef typename std::conditional<GATE, float, TOut>::type stage_t;
    stage_t* sO = reinterpret_cast<stage_t*>(smem + Lay::O_A);
    constexpr int LDO = DVS + 16 / (int)sizeof(stage_t);
    static_assert(kC * LDO * (int)sizeof(stage_t) <= Lay::SZ_AW, "O staging");
    {
      f32x4 y[NJW];
#pragma unroll
      for (int j = 0; j < NJW; ++j) {
        y[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        Oacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int kk = 0; kk < DK; kk += KS) {
        const frag aKc = M::ld(sKc + (16 * rt + l16) * LDK + kk + kofs);
        const frag aQc = M::ld(sQc + (16 * rt + l16) * LDK + kk + kofs);
#pragma unroll
        for (int j = 0; j < NJW; ++j) {
          const frag bS = M::ld(sST + (16 * (jt0 + j) + l16) * LDK + kk + kofs);
          y[j] = M::mma(aKc, bS, y[j]);
          Oacc[j] = M::mma(aQc, bS, Oacc[j]);
        }
      }
      const int i0 = 16 * rt + 4 * lg;
      const f32x4 brow = *reinterpret_cast<const f32x4*>(sBeta + i0);
#pragma unroll
      for (int j = 0; j < NJW; ++j) {
        const int jv = 16 * (jt0 + j) + l16;
        f32x4 z;
#pragma unroll
        for (int m = 0; m < 4; ++m) z[m] = brow[m] * (to_f32(sV[(i0 + m) * LDV + jv]) - y[j][m]);
        *reinterpret_cast<f32x4*>(sZT + jv * LDZ + i0) = z;
      }
    }
    __syncthreads();

    prefetch(tn, 3);
    // ---- U = (I + A)^-1 Diag(beta) Z by block forward substitution over the four
    // row tiles, U_R = D_R (beta Z_R - sum_{J<R} A_RJ U_J): one wave per value-column
    // tile, all in float32 MFMA from registers (no triangular factor is formed).
    // Each wave reads its whole column tile of Z before writing U over it.
    if (wave < NJT) {
      __builtin_amdgcn_s_setprio(2);  // the substitution chains are this phase's critical path
      const int jt = wave, jv = 16 * jt + l16;
      // the left operands, in the transposed result layout: lane holds X[l16][4 lg + kb]
      auto left = [&](const float* X, int ldx, int rx, int cx) {
        return *reinterpret_cast<const f32x4*>(X + (rx + l16) * ldx + cx + 4 * lg);
      };
      auto mul = [&](const f32x4& Xt, const f32x4& Y, f32x4 acc) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc = mma_f32(Xt[kb], Y[kb], acc);
        return acc;
      };
      f32x4 acc[kNSub];  // beta Z_R, then minus the terms of the row tiles already solved
      f32x4 dl[kNSub], al[6];  // D_R and A_RJ (J < R), loaded before the chain starts
#pragma unroll
      for (int R = 0; R < kNSub; ++R) {
        acc[R] = *reinterpret_cast<const f32x4*>(sZT + jv * LDZ + kSub * R + 4 * lg);
        dl[R] = left(sD, LDD, kSub * R, 0);
      }
#pragma unroll
      for (int R = 1, n = 0; R < kNSub; ++R)
#pragma unroll
        for (int J = 0; J < R; ++J, ++n) al[n] = left(sA, LDA, kSub * R, kSub * J);
      // U (operand type) overwrites Z (float) in these rows: keep every Z load ahead of
      // the stores (the wave's shared-memory accesses then execute in program order)
      asm volatile("" ::: "memory");
      // right-looking: once U_J is known its term goes into every later row tile, so
      // the chain through the four tiles is one product per step
#pragma unroll
      for (int J = 0; J < kNSub; ++J) {
        const f32x4 u = mul(dl[J], acc[J], f32x4{0.f, 0.f, 0.f, 0.f});
        const f32x4 nu = -u;
#pragma unroll
        for (int R = J + 1; R < kNSub; ++R) acc[R] = mul(al[R * (R - 1) / 2 + J], nu, acc[R]);
        const int i0 = kSub * J + 4 * lg;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const op_t uh = from_f32<op_t>(u[m]);
          sUT[jv * LDU + i0 + m] = uh;
          if constexpr (BF16) sUT2[jv * LDU + i0 + m] = from_f32<op_t>(u[m] - to_f32(uh));
        }
      }
      __builtin_amdgcn_s_setprio(0);
    } else if (BF16 && wave >= 4) {
      // meanwhile: P (float32) -> hi / lo bfloat16 operand rows in place (hi at element
      // 0 of the row, lo at element kC); a wave owns whole rows, four lanes per row, so
      // a row's loads all precede its stores
      const int r = 16 * (wave - 4) + (lane >> 2), c = 16 * (lane & 3);
      float pf[16];
      load8(sP + r * LDA + c, pf);
      load8(sP + r * LDA + c + 8, pf + 8);
      typedef typename Mfma<true>::frag bfrag;
      bfrag h[2], l[2];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const __bf16 hh_ = (__bf16)pf[e];
        h[e / 8][e % 8] = hh_;
        l[e / 8][e % 8] = (__bf16)(pf[e] - (float)hh_);
      }
      asm volatile("" ::: "memory");
      __bf16* row = reinterpret_cast<__bf16*>(sP + r * LDA);
      *reinterpret_cast<bfrag*>(row + c) = h[0];
      *reinterpret_cast<bfrag*>(row + c + 8) = h[1];
      *reinterpret_cast<bfrag*>(row + kC + c) = l[0];
      *reinterpret_cast<bfrag*>(row + kC + c + 8) = l[1];
    }
    __syncthreads();

    // ---- O += P U (lower-triangular P), output; S <- Diag(2^G_end) S + Kbar^T U
    {
      frag ph[NKT], pl[NKT];
#pragma unroll
      for (int q = 0; q < NKT; ++q) {
        if (q * KS < kend) {
          const int k0 = q * KS + kofs;
          if constexpr (BF16) {
            const op_t* row = reinterpret_cast<const op_t*>(sP + (16 * rt + l16) * LDA);
            ph[q] = M::ld(row + k0);
            pl[q] = M::ld(row + kC + k0);
          } else {
            ph[q] = sP[(16 * rt + l16) * LDA + k0];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < NJW; ++j) {
        const int jt = jt0 + j;
        f32x4 acc = Oacc[j];
#pragma unroll
        for (int q = 0; q < NKT; ++q) {
          if (q * KS < kend) {
            const int k0 = q * KS + kofs;
            const frag uh = M::ld(sUT + (16 * jt + l16) * LDU + k0);
            acc = M::mma(ph[q], uh, acc);
            if constexpr (BF16) {
              const frag ul = M::ld(sUT2 + (16 * jt + l16) * LDU + k0);
              acc = M::mma(pl[q], uh, acc);
              acc = M::mma(ph[q], ul, acc);
            }
          }
        }
        // O tile -> shared memory (A/W slot, free after the row-tile phase)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          sO[(16 * rt + 4 * lg + m) * LDO + 16 * jt + l16] = from_f32<stage_t>(acc[m]);
      }
    }
    {
      static_assert(NW % NJT == 0, "whole value-column tiles per wave");
      // this wave's value-column tile of U, read once for its SPW key-channel tiles
      const int jt = wave % NJT;
      frag uh[NKT], ul[NKT];
#pragma unroll
      for (int q = 0; q < NKT; ++q) {
        uh[q] = M::ld(sUT + (16 * jt + l16) * LDU + q * KS + kofs);
        if constexpr (BF16) ul[q] = M::ld(sUT2 + (16 * jt + l16) * LDU + q * KS + kofs);
      }
#pragma unroll
      for (int i = 0; i < SPW; ++i) {
        const int ct = (wave / NJT) * SPW + i;
        const f32x4 gam = *reinterpret_cast<const f32x4*>(sEGam + 16 * ct + 4 * lg);
        f32x4 s = Sacc[i] * gam;
#pragma unroll
        for (int q = 0; q < NKT; ++q) {
          const frag ak = M::ld(sKbT + (16 * ct + l16) * LDC + q * KS + kofs);
          s = M::mma(ak, uh[q], s);
          if constexpr (BF16) s = M::mma(ak, ul[q], s);
        }
        Sacc[i] = s;
#pragma unroll
        for (int m = 0; m < 4; ++m) rc.finite(s[m], kRangeState);
      }
    }
    store_state_operand();  // only the row-tile phase reads it, and that phase is over
    __syncthreads();
    if (GATE && emit) {
      // gated output: o * sigmoid(z) for this thread's unit of 8 values, rounded once
      const int64_t ob = ((b * T + t0) * H + h) * DV + j0;
      const int nvalid = (int)((te - t0) < kC ? (te - t0) : kC);
      const int r = tid / GU, c = (tid % GU) * 8;
      if (tid < kC * GU && r < nvalid) {
        float z[8], y[8];
        if constexpr (sizeof(TIn) == 2) {
          unpack16(pz[0], (TIn*)nullptr, z);
        } else {
          unpack16(pz[0], (TIn*)nullptr, z);
          unpack16(pz[GPC - 1], (TIn*)nullptr, z + 4);
        }
        const float* so = reinterpret_cast<const float*>(sO) + r * LDO + c;
        const f32x4 y0 = *reinterpret_cast<const f32x4*>(so);
        const f32x4 y1 = *reinterpret_cast<const f32x4*>(so + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y[e] = y0[e] * sigmoid_hw(z[e]);
          y[4 + e] = y1[e] * sigmoid_hw(z[4 + e]);
        }
        const uint32_t off = ((uint32_t)r * rs_v + (uint32_t)c) * (uint32_t)sizeof(TOut);
        if constexpr (sizeof(TOut) == 2) {
          bf16x8 w;
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = (__bf16)y[e];
          st_at<bf16x8>(go + ob, off, w);
        } else {
          st_at<f32x4>(go + ob, off, f32x4{y[0], y[1], y[2], y[3]});
          st_at<f32x4>(go + ob, off + 16u, f32x4{y[4], y[5], y[6], y[7]});
        }
      }
    } else if (emit) {  // output: one 16-byte store per piece, rows of DVS contiguous values
      constexpr int PPR = DVS * (int)sizeof(TOut) / 16;  // 16-byte pieces per row
      const int64_t ob = ((b * T + t0) * H + h) * DV + j0;
      const int nvalid = (int)((te - t0) < kC ? (te - t0) : kC);
#pragma unroll
      for (int it = 0; it < (kC * PPR + NT - 1) / NT; ++it) {
        const int pc = tid + NT * it;
        const int r = pc / PPR, c = (pc % PPR) * (16 / (int)sizeof(TOut));
        if (pc >= kC * PPR) break;
        if (r < nvalid)
          st_at<uint4>(go + ob, ((uint32_t)r * rs_v + (uint32_t)c) * (uint32_t)sizeof(TOut),
                       *reinterpret_cast<const uint4*>(sO + r * LDO + c));
      }
    }

    stage(tn);

    // checkpoint: every ck_every tokens, or at the listed positions (ck_pos)
    int64_t ck_idx = -1, nck = 0;
    if (emit && p.ck) {
      const int64_t end = t0 + kC;  // tokens consumed after this chunk
      if (p.ck_pos) {
        while (ck_next < p.n_ck && p.ck_pos[ck_next] < end) ++ck_next;
        if (ck_next < p.n_ck && p.ck_pos[ck_next] == end && end <= te) ck_idx = ck_next++;
        nck = p.n_ck;
      } else if (end % p.ck_every == 0 && end <= te) {
        nck = T / p.ck_every;
        ck_idx = end / p.ck_every - 1;
      }
    }
    if (ck_idx >= 0) {
      float* dst = p.ck + ((b * nck + ck_idx) * H + h) * (int64_t)DK * DV;
#pragma unroll
      for (int i = 0; i < SPW; ++i) {
        const int ct = (wave / NJT) * SPW + i, jt = wave % NJT;
#pragma unroll
        for (int m = 0; m < 4; ++m)
          dst[(int64_t)(16 * ct + 4 * lg + m) * DV + j0 + 16 * jt + l16] = Sacc[i][m];
      }
    }
    __syncthreads();
  }

  // state at the end of the walk: the final state (last segment of mode 0), or
  // the segment summary (mode 1; transitions have row stride DK)
  float* dst = nullptr;
  int64_t ld = DV;
  if (p.mode == 0) {
    if (seg == p.nseg - 1 && p.s_final) dst = p.s_final + head_off;
  } else if (pmode) {
    dst = p.seg_p + seg_unit * DK * DK;
    ld = DK;
  } else {
    dst = p.seg_z + seg_unit * DK * DV;
  }
  if (dst) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int ct = (wave / NJT) * SPW + i, jt = wave % NJT;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        dst[(int64_t)(16 * ct + 4 * lg + m) * ld + j0 + 16 * jt + l16] = Sacc[i][m];
    }
  }
}

template <typename TIn, typename TOut, int DK, int DV, int DVS>
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  typedef PrefillLayout<TIn, DK, DVS> Lay;
  auto kern = a.ogate ? chunk_fwd_kernel<TIn, TOut, DK, DV, DVS, true>
                      : chunk_fwd_kernel<TIn, TOut, DK, DV, DVS, false>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     Lay::TOTAL);
  if (e != hipSuccess) return e;
  constexpr int NSLICE = DV / DVS, NPSL = DK / DVS;
  const int64_t units = a.B * (a.nseg > 1 ? a.nseg - 1 : 1) * a.H;
  const int64_t grid = prefill_grid(units, a.mode ? NSLICE + NPSL : NSLICE);
  kern<<<dim3((unsigned)grid), dim3(512), Lay::TOTAL, stream>>>(a);
  return hipGetLastError();
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
