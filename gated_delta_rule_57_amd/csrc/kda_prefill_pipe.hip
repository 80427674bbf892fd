// Chunked KDA forward (prefill) with 32- or 16-token chunks, pipelined inside one
// workgroup: eight "producer" waves build the state-independent operands of chunk n+1
// while four "consumer" waves run the state-dependent chain of chunk n (twelve waves,
// three per SIMD: one consumer and two producers).  One workgroup per (batch row, head,
// 64-column slice of the value dimension), bfloat16 inputs.
//
// Method (chunk of C = 16 NSUB tokens, 16-token sub-tiles R; log-decays in base-2 units,
// gamma = clamp(g) log2(e), e = 2^gamma per token and channel):
//   L_r    inclusive cumulative gamma inside r's sub-tile;  tau_R = 2^(sub-tile total)
//   G_r    = ref_R + L_r, ref_R the chunk-relative start of sub-tile R
//   A[r,i] = beta_r sum_c k_rc k_ic 2^(G_rc - G_ic)      i < r
//   P[r,i] =        sum_c q_rc k_ic 2^(G_rc - G_ic)      i <= r
//   T'     = (I + A)^-1 Diag(beta)                (UT / WY form of the delta rule)
//   W      = T' Kc,  U0 = T' V                    (Kc = k 2^G)
//   U      = U0 - W S                             (S = state entering the chunk)
//   O      = Qc S + P U                           (Qc = q 2^G)
//   S'     = Diag(2^G_end) S + Kbar^T U           (Kbar = k 2^(G_end - G))
// A and P come from 16x16 tile pairs of dense bfloat16 products of a row operand
// x 2^L (<= 1) and a column operand k 2^-L; on a diagonal tile the column factor
// reaches 2^(16 * 5 log2 e) = e^80 ~ 5.5e34, inside bfloat16's range, so diagonal tiles
// are the same dense product as the others followed by a triangular mask: the
// consequence of the -5 log-decay floor that the orkas.ai blog "Kimi K3 architecture"
// draws in "A lower bound that deleted a GPU code path".  The chunk-parallel rewrite is
// the one the Towards-AI article's "Kimi Delta Attention (KDA)" section refers to, and
// the overlap of intra-chunk work with the cross-chunk state chain is the one that
// article's infrastructure section credits to K3's own kernel.
//
// Only W S, U, P U and Kbar^T U depend on the state.  Each consumer wave owns one
// 16-column tile J of the slice and keeps its d_k x 16 block of S in MFMA accumulators
// for the whole sequence.  Every product of that chain takes its state-side operand
// from registers: an MFMA result tile (lane l holds rows 4(l>>4)+m, column l&15) is
// already the right-hand operand of the next product when that product's k index runs
// over the result's rows, with the k order permuted the same way in both operands (two
// 16-row tiles per 32-wide k step, "paired tiles" below).  So the chain has no shared-
// memory round trip and no barrier of its own; the producer writes its operands in
// the matching order.
//
// Schedule of one cycle (three workgroup barriers; consumers run chunk n, producers
// build chunk n+1):
//   I1  consumers: S to bfloat16 operands, W S and Qc S, U = U0 - W S,
//       O = Qc S + P U (to staging)
//       producers: gate, decay products and operands of chunk n+1 (one wave per
//       sub-tile and quarter of the key channels); next chunk's loads issued
//   I2  consumers: S <- 2^G_end S + Kbar^T U; checkpoints
//       producers: Kc, Qc of chunk n+1 (second sub-tile's waves); two waves invert
//       I + A_RR, two build P
//   I3  consumers: output stores
//       producers: T' from the inverses, W and U0, Kbar and 2^G_end of chunk n+1
// Every array the consumers read for chunk n is written for chunk n+1 in a later
// interval than the one that reads it, so one buffer of each suffices.
//
// Precision (bfloat16 inputs, float32 accumulation): P's diagonal tiles, U, S, Kbar and
// T' are carried as hi + lo bfloat16 pairs; A, W, Qc, Kc and V as single bfloat16;
// the 16x16 inverses and the off-diagonal block of T' are float32 MFMA products.

#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace pipe {

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// hi + lo bfloat16 parts of four floats (hi rounded to nearest, lo = x - hi rounded)
struct HL4 {
  bf16x4 h, l;
};
__device__ __forceinline__ HL4 split4(f32x4 x) {
  HL4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.h[i] = (__bf16)x[i];
    r.l[i] = (__bf16)(x[i] - (float)r.h[i]);
  }
  return r;
}
__device__ __forceinline__ bf16x4 hi4(f32x4 x) {
  bf16x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (__bf16)x[i];
  return r;
}

// acc + X Y for 16x16 float32 matrices in the MFMA result layout, X passed transposed
// (Xt) and Y as is, on the float32 MFMA (16x16x4, four k steps): lane l's value m of Xt
// is X[l&15][4(l>>4)+m] and its value m of Y is Y[4(l>>4)+m][l&15], both belonging to
// k = 4(l>>4)+m, which is k step m and k index l>>4 of that step in both operands.
__device__ __forceinline__ f32x4 mmf(f32x4 Xt, f32x4 Y, f32x4 acc) {
#pragma unroll
  for (int m = 0; m < 4; ++m) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Xt[m], Y[m], acc, 0, 0, 0);
  return acc;
}

// Position of token t (0..31) inside a 32-wide k step in "paired tile" order: the k
// slots 8j..8j+7 of a 16x16x32 product hold rows 4j..4j+3 of tile 0 and then of tile 1,
// the order of two result tiles used as an operand.
__device__ __forceinline__ int pt_pos(int t) { return 8 * ((t & 15) >> 2) + 4 * (t >> 4) + (t & 3); }

template <int DK, int NSUB>
struct PipeLayout {
  static constexpr int C = 16 * NSUB;
  static constexpr int LDK = DK + 8;  // [token][channel] bfloat16 rows
  static constexpr int LDT = 32 + 8;  // [x][32 token positions] bfloat16 rows
  static constexpr int LDO = 64 + 4;  // output staging, float32
  // consumer-facing arrays (written for chunk n+1 while chunk n is consumed)
  static constexpr int O_W = 0;                                  // W [C][LDK], channel-paired order
  static constexpr int O_QC = O_W + C * LDK * 2;                 // Qc, same layout
  static constexpr int O_U0 = O_QC + C * LDK * 2;                // U0 fragments [NSUB][4][64] f32x4
  static constexpr int O_PH = O_U0 + NSUB * 4 * 64 * 16;         // P hi [C][LDT] (paired tokens)
  static constexpr int O_PL = O_PH + C * LDT * 2;                // P lo
  static constexpr int O_KBH = O_PL + C * LDT * 2;               // Kbar^T hi [DK][LDT]
  static constexpr int O_KBL = O_KBH + DK * LDT * 2;             // Kbar^T lo
  static constexpr int O_GAM = O_KBL + DK * LDT * 2;             // 2^G_end [DK] f32
  // producer scratch
  static constexpr int O_KR = O_GAM + DK * 4;                    // k 2^L [C][LDK]
  static constexpr int O_QH = O_KR + C * LDK * 2;                // q 2^L hi
  static constexpr int O_QL = O_QH + C * LDK * 2;                // q 2^L lo
  static constexpr int O_KDH = O_QL + C * LDK * 2;               // k 2^-L hi
  static constexpr int O_KDL = O_KDH + C * LDK * 2;              // k 2^-L lo
  static constexpr int O_KS = O_KDL + C * LDK * 2;               // k 2^(tau_0 - L), rows 0..15
  static constexpr int O_KCT = O_KS + (NSUB == 2 ? 32 * LDK * 2 : 0);  // Kc^T [DK][LDT]
  static constexpr int O_VT = O_KCT + DK * LDT * 2;              // V^T slice [64][LDT]
  static constexpr int O_TF = O_VT + 64 * LDT * 2;               // inverse fragments [5][64] f32x4
  static constexpr int O_BETA = O_TF + 5 * 64 * 16;              // beta [32] f32
  static constexpr int O_TAU = O_BETA + 32 * 4;                  // tau [2][DK] f32
  // consumer staging
  static constexpr int O_O = O_TAU + 2 * DK * 4;                 // O [C][LDO] f32
  static constexpr int TOTAL = O_O + C * LDO * 4;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
  static_assert(O_KR % 16 == 0 && O_KCT % 16 == 0 && O_TF % 16 == 0 && O_O % 16 == 0 &&
                    O_U0 % 16 == 0 && O_PH % 16 == 0 && O_KBH % 16 == 0 && TOTAL % 16 == 0,
                "16-byte aligned arrays");
};

constexpr int kPipeThreads = 768;  // 4 consumer + 8 producer waves

template <typename TOut, int DK, int DV, int NSUB, bool GATE>
__global__ void __launch_bounds__(kPipeThreads) chunk_pipe_kernel(PrefillArgs p) {
  typedef PipeLayout<DK, NSUB> Lay;
  typedef __bf16 TIn;
  constexpr int C = Lay::C, LDK = Lay::LDK, LDT = Lay::LDT, LDO = Lay::LDO;
  constexpr int DVS = 64, NSLICE = DV / DVS, NPSL = DK / DVS;
  constexpr int NCT = DK / 16;  // state tiles per consumer wave (key channels / 16)
  constexpr int NKS = DK / 32;  // 32-wide k steps over the key channels
  static_assert(DK % 64 == 0 && DV % 64 == 0, "head dimensions");

  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* sW = reinterpret_cast<__bf16*>(smem + Lay::O_W);
  __bf16* sQc = reinterpret_cast<__bf16*>(smem + Lay::O_QC);
  f32x4* sU0 = reinterpret_cast<f32x4*>(smem + Lay::O_U0);
  __bf16* sPh = reinterpret_cast<__bf16*>(smem + Lay::O_PH);
  __bf16* sPl = reinterpret_cast<__bf16*>(smem + Lay::O_PL);
  __bf16* sKbh = reinterpret_cast<__bf16*>(smem + Lay::O_KBH);
  __bf16* sKbl = reinterpret_cast<__bf16*>(smem + Lay::O_KBL);
  float* sGam = reinterpret_cast<float*>(smem + Lay::O_GAM);
  __bf16* sKr = reinterpret_cast<__bf16*>(smem + Lay::O_KR);
  __bf16* sQh = reinterpret_cast<__bf16*>(smem + Lay::O_QH);
  __bf16* sQl = reinterpret_cast<__bf16*>(smem + Lay::O_QL);
  __bf16* sKdh = reinterpret_cast<__bf16*>(smem + Lay::O_KDH);
  __bf16* sKdl = reinterpret_cast<__bf16*>(smem + Lay::O_KDL);
  __bf16* sKs = reinterpret_cast<__bf16*>(smem + Lay::O_KS);
  __bf16* sKcT = reinterpret_cast<__bf16*>(smem + Lay::O_KCT);
  __bf16* sVT = reinterpret_cast<__bf16*>(smem + Lay::O_VT);
  f32x4* sTF = reinterpret_cast<f32x4*>(smem + Lay::O_TF);
  float* sBeta = reinterpret_cast<float*>(smem + Lay::O_BETA);
  float* sTau = reinterpret_cast<float*>(smem + Lay::O_TAU);
  float* sO = reinterpret_cast<float*>(smem + Lay::O_O);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool consumer = wave < 4;
  // Lane indices, refreshed at the top of every interval: the per-lane shared-memory
  // addresses derived from them are then recomputed inside the loop (a few adds)
  // instead of being hoisted out of it and held in registers across it.
  int tid = threadIdx.x, lane, c16, lg, cp, q1, c0, tr0, jp, tq;

  // ---- workgroup -> (unit, slice), unit = (b, segment, h); all slices of a unit on one
  // XCD (consecutive workgroups go round-robin to the 8 XCDs).  Segment path as in the
  // 64-token kernel: mode 1 summarises segments 0..nseg-2 (Z from zero / the initial
  // state, P from the identity with v = 0), mode 0 runs segments from their entry states.
  const int nsl = p.mode ? NSLICE + NPSL : NSLICE;
  const int64_t nsg = p.nseg > 1 ? p.nseg - 1 : 1;
  const int64_t seg0 = (p.mode == 0 && p.nseg > 1) ? 1 : 0;
  const int64_t x = blockIdx.x;
  const int64_t grp = x / (8 * nsl);
  const int gi = (int)(x % (8 * nsl));
  const int64_t unit = grp * 8 + (gi % 8);
  const int slice = gi / 8;
  if (unit >= p.B * nsg * p.H) return;
  const int64_t h = unit % p.H, bj = unit / p.H, seg = bj % nsg + seg0, b = bj / nsg;
  const bool pmode = slice >= NSLICE;
  if (pmode && seg == 0) return;
  const int j0 = (pmode ? slice - NSLICE : slice) * DVS;
  const int64_t T = p.T, H = p.H;
  const RangeCheck rc{p.range_flags};  // checks only in a KDA_DEBUG_RANGE build
  const int64_t tb = seg * p.seg_len;
  const int64_t te = (T - tb) < p.seg_len ? T : tb + p.seg_len;
  const bool emit = p.mode == 0 || (seg == 0 && !pmode);
  const int64_t nchunks = (te - tb + C - 1) / C;

  const TIn* gq = reinterpret_cast<const TIn*>(p.q);
  const TIn* gk = reinterpret_cast<const TIn*>(p.k);
  const TIn* gv = reinterpret_cast<const TIn*>(p.v);
  const TIn* gg = reinterpret_cast<const TIn*>(p.g);
  const TIn* gb = reinterpret_cast<const TIn*>(p.beta);
  TOut* go = reinterpret_cast<TOut*>(p.o);
  const int64_t head_off = (b * H + h) * (int64_t)DK * DV;
  const int64_t seg_unit = (b * p.nseg + seg) * H + h;
  const uint32_t rs_k = (uint32_t)(H * DK), rs_v = (uint32_t)(H * DV);

  // shared memory starts at zero: positions no chunk writes (the upper block of P, the
  // second token tile of 16-token chunks) must read as zero
  for (int i = tid; i < Lay::TOTAL / 16; i += kPipeThreads)
    reinterpret_cast<uint4*>(smem)[i] = make_uint4(0u, 0u, 0u, 0u);

  // ======================= producer-side per-lane constants =======================
  // Operand prep: producer wave pw (0..7) takes sub-tile R1 = pw >> 2 and key channels
  // 32 cq .. +31, cq = pw & 3; lane = (channel pair cp = lane & 15, 4-token range
  // q1 = lane >> 4): channels c0 = 32 cq + 2 cp and c0 + 1, tokens tr0 = 16 R1 + 4 q1 ..
  // tr0 + 3 (chunk-relative).  v: lane (value-column pair jp, 4-token group tq) of the
  // 256 lanes of producer waves 0..3.
  const int pw = wave - 4;
  const int R1 = (pw >> 2) & 1, cq = pw & 3;
  const bool act1 = !consumer && R1 < NSUB && 32 * cq < DK;
  auto refresh = [&]() {
    asm volatile("" : "+v"(tid));
    lane = tid & 63;
    c16 = lane & 15;
    lg = lane >> 4;
    cp = lane & 15;
    q1 = lane >> 4;
    c0 = 32 * cq + 2 * cp;
    tr0 = 16 * R1 + 4 * q1;
    const int vtid = (pw & 3) * 64 + lane;
    jp = vtid & 31;
    tq = vtid >> 5;
  };
  refresh();
  // tq = 2 pw + (lane >> 5): the 4-token groups of a chunk are tq < C / 4, whole waves
  const bool actv = !consumer && !pmode && pw < 4 && 8 * pw < C;

  uint32_t rk[4], rq[4], rg[4], rv[4];
  TIn rb = (TIn)0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) rk[j] = rq[j] = rg[j] = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) rv[i] = 0u;

  // raw inputs of the chunk starting at t0c into registers (rows past the end of the
  // walk load the last valid token, in bounds; they are masked when used)
  auto prefetch = [&](int64_t t0c) {
    const int last = (int)((te - t0c) < C ? (te - t0c) : C) - 1;
    const int64_t cb = (b * T + t0c) * H + h;
    if (act1) {
      const TIn* kb = gk + cb * DK;
      const TIn* qb = gq + cb * DK;
      const TIn* gb2 = gg + cb * DK;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t off = ((uint32_t)min(tr0 + j, last) * rs_k + (uint32_t)c0) * 2u;
        rk[j] = ld_at<uint32_t>(kb, off);
        rq[j] = ld_at<uint32_t>(qb, off);
        rg[j] = ld_at<uint32_t>(gb2, off);
      }
    }
    if (actv) {
      const TIn* vb = gv + cb * DV + j0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        rv[i] = ld_at<uint32_t>(vb, ((uint32_t)min(4 * tq + i, last) * rs_v + (uint32_t)(2 * jp)) * 2u);
    }
    if (!consumer && pw == 0 && lane < C)
      rb = ld_at<TIn>(gb + cb, (uint32_t)min(lane, last) * (uint32_t)H * 2u);
  };

  // k 2^L, q 2^L and k 2^-L of this lane's 4 tokens x 2 channels, held from the operand
  // step (I1) to the steps that form Kc, Qc (I2) and Kbar (I3) (the producer loop's
  // registers are its own)
  f32x2 hkr[4], hqr[4], hkd[4];
  f32x2 htau = {1.f, 1.f};  // this lane's sub-tile total 2^(tau) of its two channels

  // ---- I1 producer step: gate, decay products, operands of the chunk at t0c
  auto produce_operands = [&](int64_t t0c) {
    const int nvalid = (int)((te - t0c) < C ? (te - t0c) : C);
    if (act1) {
      // per-token decays 2^gamma (1 on padded rows); the branch on the gate form is
      // outside the token loop, so that each form is one straight run of code
      f32x2 e[4];
      if (p.gate_logits) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x2 a = unpack2(rg[j]);
          e[j] = f32x2{exp2_hw(gamma_from_logit(a.x)), exp2_hw(gamma_from_logit(a.y))};
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x2 gg2 = unpack2(rg[j]);
          e[j] = f32x2{exp2_hw(clamp_log_decay(gg2.x) * kLog2e),
                       exp2_hw(clamp_log_decay(gg2.y) * kLog2e)};
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (tr0 + j >= nvalid) e[j] = f32x2{1.f, 1.f};
      // prefix products over the range; the sub-tile's earlier ranges (lanes 16 and 32
      // apart hold the same channels) by an exclusive scan over the four ranges
      f32x2 pre[4];
      pre[0] = e[0];
#pragma unroll
      for (int j = 1; j < 4; ++j) pre[j] = pre[j - 1] * e[j];
      const f32x2 own = pre[3];
      const f32x2 t1 = {__shfl_xor(own.x, 16, 64), __shfl_xor(own.y, 16, 64)};
      const f32x2 p01 = own * t1;  // product of this range pair (ranges 0-1 or 2-3)
      const f32x2 t2 = {__shfl_xor(p01.x, 32, 64), __shfl_xor(p01.y, 32, 64)};
      f32x2 off = (q1 & 1) ? t1 : f32x2{1.f, 1.f};
      if (q1 & 2) off *= t2;
      htau = p01 * t2;
      // 2^-L at the range's last token: the reciprocal (1 ulp) of its prefix; a sub-tile's
      // product stays >= 2^(-16 * 5 log2 e), a normal float.  Then suffix products.
      const f32x2 po = off * own;
      f32x2 em = {__builtin_amdgcn_rcpf(po.x), __builtin_amdgcn_rcpf(po.y)};
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        const bool valid = tr0 + j < nvalid;
        const uint32_t msk = valid ? 0xffffffffu : 0u;
        const f32x2 kf = unpack2(rk[j] & msk), qf = unpack2(rq[j] & msk);
        const f32x2 ep = off * pre[j];
        const int r = tr0 + j;
        const f32x2 kr = kf * ep, qr = qf * ep, kd = kf * em;
        rc.factors(ep.x, em.x);
        rc.factors(ep.y, em.y);
        rc.operand(kr.x, kBf16Max), rc.operand(kr.y, kBf16Max), rc.operand(qr.x, kBf16Max);
        rc.operand(qr.y, kBf16Max), rc.operand(kd.x, kBf16Max), rc.operand(kd.y, kBf16Max);
        hkr[j] = kr;
        hqr[j] = qr;
        hkd[j] = kd;
        em *= e[j];
        *reinterpret_cast<uint32_t*>(sKr + r * LDK + c0) = pack2(kr, (uint32_t*)nullptr);
        const uint32_t qh = pack2(qr, (uint32_t*)nullptr);
        *reinterpret_cast<uint32_t*>(sQh + r * LDK + c0) = qh;
        *reinterpret_cast<uint32_t*>(sQl + r * LDK + c0) = pack2(qr - unpack2(qh), (uint32_t*)nullptr);
        const uint32_t kh = pack2(kd, (uint32_t*)nullptr);
        *reinterpret_cast<uint32_t*>(sKdh + r * LDK + c0) = kh;
        *reinterpret_cast<uint32_t*>(sKdl + r * LDK + c0) = pack2(kd - unpack2(kh), (uint32_t*)nullptr);
        if constexpr (NSUB == 2) {
          // sub-tile 0's column operand of the off-diagonal tile pair (1, 0):
          // k 2^(tau_0 - L) <= 1 (sub-tile 1's lanes write rows 16..31 of the array,
          // never read, which keeps this loop free of branches)
          *reinterpret_cast<uint32_t*>(sKs + r * LDK + c0) = pack2(kd * htau, (uint32_t*)nullptr);
        }
      }
      if (q1 == 0) *reinterpret_cast<f32x2*>(sTau + R1 * DK + c0) = htau;
    }
    if (actv) {
      // V^T slice in paired-tile token order; four tokens are one 4-group
      uint32_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;  // columns 2jp (w0, w1), 2jp+1 (w2, w3)
      uint32_t v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (4 * tq + i < nvalid) ? rv[i] : 0u;
      w0 = (v[0] & 0xffffu) | (v[1] << 16);
      w1 = (v[2] & 0xffffu) | (v[3] << 16);
      w2 = (v[0] >> 16) | (v[1] & 0xffff0000u);
      w3 = (v[2] >> 16) | (v[3] & 0xffff0000u);
      const int pos = pt_pos(4 * tq);
      *reinterpret_cast<uint2*>(sVT + (2 * jp) * LDT + pos) = make_uint2(w0, w1);
      *reinterpret_cast<uint2*>(sVT + (2 * jp + 1) * LDT + pos) = make_uint2(w2, w3);
    }
    if (!consumer && pw == 0 && lane < 32)
      sBeta[lane] = (lane < nvalid) ? to_f32(rb) : 0.f;
  };

  // ---- I2 producer step, part 1: Kc^T (paired token order) and Qc (paired channel
  // order) of the chunk whose operands were just built.  With two sub-tiles the second
  // sub-tile's waves do both (the first sub-tile's waves are the ones that invert and
  // build P in this interval).
  auto produce_kc_qc = [&]() {
    if (!act1) return;
    if (NSUB == 2 && R1 == 0) return;
    const int pc = 32 * (c0 >> 5) + 8 * ((c0 & 15) >> 2) + 4 * ((c0 >> 4) & 1) + (c0 & 3);
    // Kc^T rows c0, c0 + 1: four tokens from row t are one 4-group of the paired order
    auto kct = [&](const uint32_t (&kc)[4], int t) {
      const int pos = pt_pos(t);
      const uint32_t a0 = (kc[0] & 0xffffu) | (kc[1] << 16);
      const uint32_t a1 = (kc[2] & 0xffffu) | (kc[3] << 16);
      const uint32_t b0 = (kc[0] >> 16) | (kc[1] & 0xffff0000u);
      const uint32_t b1 = (kc[2] >> 16) | (kc[3] & 0xffff0000u);
      *reinterpret_cast<uint2*>(sKcT + c0 * LDT + pos) = make_uint2(a0, a1);
      *reinterpret_cast<uint2*>(sKcT + (c0 + 1) * LDT + pos) = make_uint2(b0, b1);
    };
    {
      // this lane's own rows: k 2^G and q 2^G = (x 2^L) 2^ref, 2^ref the product of the
      // earlier sub-tile's decays
      f32x2 ref = {1.f, 1.f};
      if (R1 == 1) ref = *reinterpret_cast<const f32x2*>(sTau + c0);
      uint32_t kc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kc[j] = pack2(hkr[j] * ref, (uint32_t*)nullptr);
        *reinterpret_cast<uint32_t*>(sQc + (tr0 + j) * LDK + pc) = pack2(hqr[j] * ref, (uint32_t*)nullptr);
      }
      kct(kc, tr0);
    }
    if constexpr (NSUB == 2) {
      // the first sub-tile's rows 4 q1 .. +3, same channels: its reference is the chunk
      // start, so Kc = k 2^L and Qc = q 2^L are the values already rounded into sKr and
      // sQh, copied into the Kc^T and Qc layouts
      const int t0 = 4 * q1;
      uint32_t kc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kc[j] = *reinterpret_cast<const uint32_t*>(sKr + (t0 + j) * LDK + c0);
        *reinterpret_cast<uint32_t*>(sQc + (t0 + j) * LDK + pc) =
            *reinterpret_cast<const uint32_t*>(sQh + (t0 + j) * LDK + c0);
      }
      kct(kc, t0);
    }
  };

  // ---- I2 producer step, part 2: tile products.  Wave R (< NSUB) inverts I + A_RR
  // (A_RR strictly lower, beta-scaled rows) by the product form
  // (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8), N^16 = 0, on the float32 MFMA, and
  // leaves in sTF, in the result layout: [0] T'_00^T = Diag(beta_0) D_0^T, [2] T'_11^T,
  // [3] D_0, [4] D_1^T, and (wave 1) [1] A_10.  Waves 2 and 3 form P's tile pairs.
  auto produce_tiles = [&]() {
    if (consumer) return;
    // one dense product over the key channels: rows of X (16 tokens from row xr0) against
    // rows of Y (16 tokens from row yr0), both [token][channel] arrays
    auto tile = [&](const __bf16* X, int xr0, const __bf16* Y, int yr0, f32x4 acc) {
#pragma unroll
      for (int kk = 0; kk < NKS; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(X + (xr0 + c16) * LDK + 32 * kk + 8 * lg);
        const bf16x8 bb = *reinterpret_cast<const bf16x8*>(Y + (yr0 + c16) * LDK + 32 * kk + 8 * lg);
        acc = mma(a, bb, acc);
      }
      return acc;
    };
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    if (pw < NSUB) {
      const int R = pw, r0 = 16 * R;
      // N = A_RR (rows r = 4lg+m, column i = c16) and its transpose, same layout
      const f32x4 na = tile(sKr, r0, sKdh, r0, z4);
      const f32x4 nt = tile(sKdh, r0, sKr, r0, z4);
      const f32x4 brow = *reinterpret_cast<const f32x4*>(sBeta + r0 + 4 * lg);
      const float bcol = sBeta[r0 + c16];
      f32x4 N, Nt, I4;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = 4 * lg + m;
        N[m] = (c16 < r) ? brow[m] * na[m] : 0.f;
        rc.finite(N[m], kRangeTile);
        Nt[m] = (r < c16) ? bcol * nt[m] : 0.f;
        I4[m] = (r == c16) ? 1.f : 0.f;
      }
      const f32x4 N2 = mmf(Nt, N, z4), N2t = mmf(N, Nt, z4);
      const f32x4 N4 = mmf(N2t, N2, z4), N4t = mmf(N2, N2t, z4);
      const f32x4 N8 = mmf(N4t, N4, z4);
      const f32x4 X1 = I4 - N, X1t = I4 - Nt;
      const f32x4 X2 = mmf(X1t, N2, X1), X2t = mmf(N2, X1t, X1t);
      const f32x4 X3 = mmf(X2t, N4, X2), X3t = mmf(N4, X2t, X2t);
      const f32x4 Dt = mmf(N8, X3t, X3t);  // D_R^T
      if (R == 0) {
        sTF[3 * 64 + lane] = mmf(X3t, N8, X3);  // D_0
        sTF[0 * 64 + lane] = Dt * brow;
      } else {
        sTF[4 * 64 + lane] = Dt;
        sTF[2 * 64 + lane] = Dt * brow;
        // A_10 = beta_r sum_c k~_r k_i 2^(tau_0 - L_i): rows r of sub-tile 1, columns i of 0
        if constexpr (NSUB == 2) sTF[1 * 64 + lane] = tile(sKr, 16, sKs, 0, z4) * brow;
      }
    } else if (pw == 2 || pw == 3) {
      // P^T tiles (rows i = 4lg+m, column r = c16) -> P hi / lo rows r, paired token order
      auto put = [&](int R, int I, f32x4 pt, bool diag) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if (diag && 4 * lg + m > c16) pt[m] = 0.f;
          rc.finite(pt[m], kRangeTile);
        }
        const HL4 s = split4(pt);
        const int pos = 8 * lg + 4 * I;
        *reinterpret_cast<bf16x4*>(sPh + (16 * R + c16) * LDT + pos) = s.h;
        *reinterpret_cast<bf16x4*>(sPl + (16 * R + c16) * LDT + pos) = s.l;
      };
      const int R = pw - 2;  // wave 2: the (0,0) tile (and (1,0)); wave 3: (1,1)
      if (R < NSUB) {
        const int r0 = 16 * R;
        f32x4 pt = tile(sKdh, r0, sQh, r0, z4);
        pt = tile(sKdh, r0, sQl, r0, pt);
        pt = tile(sKdl, r0, sQh, r0, pt);
        put(R, R, pt, true);
      }
      if constexpr (NSUB == 2) {
        if (R == 0) {
          // off-diagonal pair (1, 0): column operand k 2^(tau_0 - L) (single), row q 2^L hi
          const f32x4 pt = tile(sKs, 0, sQh, 16, z4);
          put(1, 0, pt, false);
        }
      }
    }
  };

  // ---- I3 producer step: Kbar (hi / lo, paired tokens) and 2^G_end; T' from the
  // inverses; W^T = Kc^T T'^T and U0 = T' V
  auto produce_w_u0 = [&]() {
    if (consumer) return;
    if (act1) {
      // Kbar = k 2^(G_end - G) = (k 2^-L) 2^(G_end - ref_R1)
      const f32x2 t0v = *reinterpret_cast<const f32x2*>(sTau + c0);
      const f32x2 t1v = NSUB == 2 ? *reinterpret_cast<const f32x2*>(sTau + DK + c0) : f32x2{1.f, 1.f};
      const f32x2 fac = R1 == 0 ? t0v * t1v : t1v;
      uint32_t kh[4], kl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x2 kb = hkd[j] * fac;
        kh[j] = pack2(kb, (uint32_t*)nullptr);
        kl[j] = pack2(kb - unpack2(kh[j]), (uint32_t*)nullptr);
      }
      {
        const int pos = pt_pos(tr0);
        const uint32_t* src[2] = {kh, kl};
        __bf16* dst[2] = {sKbh, sKbl};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const uint32_t* w = src[s];
          const uint32_t a0 = (w[0] & 0xffffu) | (w[1] << 16);
          const uint32_t a1 = (w[2] & 0xffffu) | (w[3] << 16);
          const uint32_t b0 = (w[0] >> 16) | (w[1] & 0xffff0000u);
          const uint32_t b1 = (w[2] >> 16) | (w[3] & 0xffff0000u);
          *reinterpret_cast<uint2*>(dst[s] + c0 * LDT + pos) = make_uint2(a0, a1);
          *reinterpret_cast<uint2*>(dst[s] + (c0 + 1) * LDT + pos) = make_uint2(b0, b1);
        }
      }
      if (R1 == 0 && q1 == 0) *reinterpret_cast<f32x2*>(sGam + c0) = t0v * t1v;
    }
    // Row tile R = pw >> 2 of T' per wave: waves 0-3 the first, waves 4-7 the second
    // (they alone form the off-diagonal block).  T'^T tiles in the result layout (rows
    // j = 4lg+m, column i = c16) make the paired-tile operand of that row tile: slots 0-3
    // the tile with j in sub-tile 0, slots 4-7 with j in sub-tile 1.
    const int R = pw >> 2;
    if (R >= NSUB) return;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    bf16x8 tph, tpl;
    if (R == 0) {
      const HL4 t00 = split4(sTF[0 * 64 + lane]);
      const bf16x4 zb = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
      tph = cat(t00.h, zb);
      tpl = cat(t00.l, zb);
    } else {
      // T'_10^T = -Diag(beta_0) D_0^T A_10^T D_1^T
      const f32x4 Z = mmf(sTF[1 * 64 + lane], sTF[4 * 64 + lane], z4);  // A_10^T D_1^T
      const f32x4 Y = mmf(sTF[3 * 64 + lane], Z, z4);                    // D_0^T Z
      const f32x4 b0r = *reinterpret_cast<const f32x4*>(sBeta + 4 * lg);
      const HL4 t10 = split4(-(Y * b0r));
      const HL4 t11 = split4(sTF[2 * 64 + lane]);
      tph = cat(t10.h, t11.h);
      tpl = cat(t10.l, t11.l);
    }
    // W^T tiles (ct, R), ct = 2 (pw & 3) + {0, 1} (for DK = 64 the first only): rows c =
    // channels, columns i = tokens; written into W's rows (tokens) at the channel-paired
    // positions of c..c+3
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int ct = (NCT == 8) ? 2 * (pw & 3) + u : (pw & 3);
      if (NCT != 8 && u == 1) break;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(sKcT + (16 * ct + c16) * LDT + 8 * lg);
      f32x4 w = mma(a, tph, z4);
      w = mma(a, tpl, w);
      const int pc = 32 * (ct >> 1) + 8 * lg + 4 * (ct & 1);
      *reinterpret_cast<bf16x4*>(sW + (16 * R + c16) * LDK + pc) = hi4(w);
    }
    // U0 tile (R, J = pw & 3): rows i, columns = value channels 16J + c16
    {
      const int J = pw & 3;
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(sVT + (16 * J + c16) * LDT + 8 * lg);
      f32x4 u = mma(tph, bv, z4);
      u = mma(tpl, bv, u);
      sU0[(R * 4 + J) * 64 + lane] = u;
    }
  };

  // ======================= consumer-side state =======================
  const int J = wave & 3;  // value-column tile of a consumer wave
  f32x4 Sacc[NCT];
  {
    const float* src = nullptr;
    if (seg > 0) {
      if (p.mode == 0) src = p.seg_in + seg_unit * DK * DV;
    } else if (p.s0) {
      src = p.s0 + head_off;
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int c = 16 * ct + 4 * lg + m, jv = 16 * J + c16;
        float s = 0.f;
        if (consumer) {
          if (pmode) s = (c == j0 + jv) ? 1.f : 0.f;
          else if (src) s = src[(int64_t)c * DV + j0 + jv];
        }
        Sacc[ct][m] = s;
      }
    }
  }
  bf16x8 Sbh[NKS], Sbl[NKS];  // S as paired-tile bfloat16 operands (hi, lo)
  auto state_operands = [&]() {
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) {
      const HL4 a = split4(Sacc[2 * kk]), c = split4(Sacc[2 * kk + 1]);
      Sbh[kk] = cat(a.h, c.h);
      Sbl[kk] = cat(a.l, c.l);
    }
  };
  bf16x8 Ubh, Ubl;  // U of the current chunk, paired token tiles

  // output gate of the chunk being consumed: one unit of 8 values per consumer lane
  // (row r = tid >> 3, columns 8 (tid & 7) .. +7 of the slice), loaded a cycle ahead
  float4 zr = make_float4(0.f, 0.f, 0.f, 0.f);
  auto load_gate = [&](int64_t t0c) {
    if constexpr (GATE) {
      if (consumer && emit && (tid >> 3) < C) {
        const int last = (int)((te - t0c) < C ? (te - t0c) : C) - 1;
        const TIn* zb = reinterpret_cast<const TIn*>(p.ogate) + ((b * T + t0c) * H + h) * DV + j0;
        zr = ld_at<float4>(zb, ((uint32_t)min(tid >> 3, last) * rs_v + (uint32_t)(8 * (tid & 7))) * 2u);
      }
    }
  };

  // ---- I1 consumer step: W S, Qc S, U, P U -> output staging
  auto consume_1 = [&]() {
    state_operands();
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 ws[NSUB], qs[NSUB];
#pragma unroll
    for (int R = 0; R < NSUB; ++R) {
      ws[R] = z4;
      qs[R] = z4;
#pragma unroll
      for (int kk = 0; kk < NKS; ++kk) {
        const bf16x8 aw = *reinterpret_cast<const bf16x8*>(sW + (16 * R + c16) * LDK + 32 * kk + 8 * lg);
        const bf16x8 aq = *reinterpret_cast<const bf16x8*>(sQc + (16 * R + c16) * LDK + 32 * kk + 8 * lg);
        ws[R] = mma(aw, Sbh[kk], ws[R]);
        ws[R] = mma(aw, Sbl[kk], ws[R]);
        qs[R] = mma(aq, Sbh[kk], qs[R]);
        qs[R] = mma(aq, Sbl[kk], qs[R]);
      }
    }
    f32x4 u[2];
#pragma unroll
    for (int R = 0; R < 2; ++R) u[R] = z4;
#pragma unroll
    for (int R = 0; R < NSUB; ++R) u[R] = sU0[(R * 4 + J) * 64 + lane] - ws[R];
    const HL4 u0 = split4(u[0]), u1 = split4(u[1]);
    Ubh = cat(u0.h, u1.h);
    Ubl = cat(u0.l, u1.l);
#pragma unroll
    for (int R = 0; R < NSUB; ++R) {
      const bf16x8 ph = *reinterpret_cast<const bf16x8*>(sPh + (16 * R + c16) * LDT + 8 * lg);
      const bf16x8 pl = *reinterpret_cast<const bf16x8*>(sPl + (16 * R + c16) * LDT + 8 * lg);
      f32x4 o = mma(ph, Ubh, qs[R]);
      o = mma(pl, Ubh, o);
      o = mma(ph, Ubl, o);
#pragma unroll
      for (int m = 0; m < 4; ++m) sO[(16 * R + 4 * lg + m) * LDO + 16 * J + c16] = o[m];
    }
  };

  // ---- I2 consumer step: S <- Diag(2^G_end) S + Kbar^T U
  auto consume_2 = [&]() {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const f32x4 gam = *reinterpret_cast<const f32x4*>(sGam + 16 * ct + 4 * lg);
      const bf16x8 kh = *reinterpret_cast<const bf16x8*>(sKbh + (16 * ct + c16) * LDT + 8 * lg);
      const bf16x8 kl = *reinterpret_cast<const bf16x8*>(sKbl + (16 * ct + c16) * LDT + 8 * lg);
      f32x4 s = Sacc[ct] * gam;
      s = mma(kh, Ubh, s);
      s = mma(kh, Ubl, s);
      s = mma(kl, Ubh, s);
      Sacc[ct] = s;
#pragma unroll
      for (int m = 0; m < 4; ++m) rc.finite(s[m], kRangeState);
    }
  };

  // ---- I3 consumer step: output rows of the chunk at t0c from staging to HBM
  auto consume_3 = [&](int64_t t0c) {
    if (!emit) return;
    const int nvalid = (int)((te - t0c) < C ? (te - t0c) : C);
    const int r = tid >> 3, c = 8 * (tid & 7);
    if (r >= nvalid) return;
    const float* so = sO + r * LDO + c;
    const f32x4 y0 = *reinterpret_cast<const f32x4*>(so);
    const f32x4 y1 = *reinterpret_cast<const f32x4*>(so + 4);
    float y[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
    if constexpr (GATE) {
      float zf[8];
      unpack16(zr, (TIn*)nullptr, zf);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] *= sigmoid_hw(zf[e]);
    }
    const int64_t ob = ((b * T + t0c) * H + h) * DV + j0;
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
  };

  // checkpoint state writes of the consumer waves (every ck_every tokens or at ck_pos)
  int64_t ck_next = 0;
  if (emit && p.ck && p.ck_pos) {
    int64_t lo = 0, hi = p.n_ck;
    while (lo < hi) {
      const int64_t mid = (lo + hi) / 2;
      if (p.ck_pos[mid] < tb + C) lo = mid + 1;
      else hi = mid;
    }
    ck_next = lo;
  }
  auto store_state = [&](float* dst, int64_t ld) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        dst[(int64_t)(16 * ct + 4 * lg + m) * ld + j0 + 16 * J + c16] = Sacc[ct][m];
  };

  // ======================= the two roles =======================
  // Producers and consumers run loops of their own with the same number of workgroup
  // barriers (one after clearing shared memory, three in the prologue, three per
  // cycle): neither role's registers then pass through the other's code, and no
  // load in flight has to be waited for where the two would merge.
  __syncthreads();  // shared memory cleared
  if (!consumer) {
    // prologue: chunk 0's operands
    prefetch(tb);
    produce_operands(tb);
    if (nchunks > 1) prefetch(tb + C);
    __syncthreads();
    produce_kc_qc();
    produce_tiles();
    __syncthreads();
    produce_w_u0();
    __syncthreads();
    for (int64_t n = 0; n < nchunks; ++n) {
      const int64_t t0 = tb + n * C;
      const bool more = n + 1 < nchunks;
      refresh();
      if (more) {
        produce_operands(t0 + C);
        if (n + 2 < nchunks) prefetch(t0 + 2 * C);
      }
      __syncthreads();
      refresh();
      if (more) {
        produce_kc_qc();
        produce_tiles();
      }
      __syncthreads();
      refresh();
      if (more) produce_w_u0();
      __syncthreads();
    }
  } else {
    load_gate(tb);
    __syncthreads();
    __syncthreads();
    __syncthreads();
    for (int64_t n = 0; n < nchunks; ++n) {
      const int64_t t0 = tb + n * C;
      refresh();
      consume_1();
      __syncthreads();
      refresh();
      consume_2();
      int64_t ck_idx = -1, nck = 0;
      if (emit && p.ck) {
        const int64_t end = t0 + C;
        if (p.ck_pos) {
          while (ck_next < p.n_ck && p.ck_pos[ck_next] < end) ++ck_next;
          if (ck_next < p.n_ck && p.ck_pos[ck_next] == end && end <= te) ck_idx = ck_next++;
          nck = p.n_ck;
        } else if (end % p.ck_every == 0 && end <= te) {
          nck = T / p.ck_every;
          ck_idx = end / p.ck_every - 1;
        }
      }
      if (ck_idx >= 0) store_state(p.ck + ((b * nck + ck_idx) * H + h) * (int64_t)DK * DV, DV);
      __syncthreads();
      refresh();
      consume_3(t0);
      if (n + 1 < nchunks) load_gate(t0 + C);
      __syncthreads();
    }
    // state at the end of the walk
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
    if (dst) store_state(dst, ld);
  }
}

template <typename TOut, int DK, int DV, int NSUB>
hipError_t launch_pipe(const PrefillArgs& a, hipStream_t stream) {
  typedef PipeLayout<DK, NSUB> Lay;
  auto kern = a.ogate ? chunk_pipe_kernel<TOut, DK, DV, NSUB, true>
                      : chunk_pipe_kernel<TOut, DK, DV, NSUB, false>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     Lay::TOTAL);
  if (e != hipSuccess) return e;
  constexpr int NSLICE = DV / 64, NPSL = DK / 64;
  const int64_t units = a.B * (a.nseg > 1 ? a.nseg - 1 : 1) * a.H;
  const int64_t grid = prefill_grid(units, a.mode ? NSLICE + NPSL : NSLICE);
  kern<<<dim3((unsigned)grid), dim3(kPipeThreads), Lay::TOTAL, stream>>>(a);
  return hipGetLastError();
}

template <typename TOut, int NSUB>
hipError_t dispatch_dims(const PrefillArgs& a, int dk, int dv, hipStream_t s) {
  if (dk == 128 && dv == 128) return launch_pipe<TOut, 128, 128, NSUB>(a, s);
  if (dk == 128 && dv == 64) return launch_pipe<TOut, 128, 64, NSUB>(a, s);
  if (dk == 64 && dv == 128) return launch_pipe<TOut, 64, 128, NSUB>(a, s);
  return launch_pipe<TOut, 64, 64, NSUB>(a, s);
}

}  // namespace pipe

hipError_t chunk_fwd_pipe(const PrefillArgs& a, int chunk, int dk, int dv, bool out_bf16,
                          hipStream_t s) {
  if (chunk == 32)
    return out_bf16 ? pipe::dispatch_dims<__bf16, 2>(a, dk, dv, s)
                    : pipe::dispatch_dims<float, 2>(a, dk, dv, s);
  return out_bf16 ? pipe::dispatch_dims<__bf16, 1>(a, dk, dv, s)
                  : pipe::dispatch_dims<float, 1>(a, dk, dv, s);
}

}  // namespace kda
