// Chunked KDA forward (prefill): one workgroup per (batch row, head, d_v slice)
// walks the sequence chunk by chunk, keeping its slice of the float32 state in
// MFMA accumulators for the whole sequence.
//
// Method (chunk of C = 64 tokens, 16-token sub-tiles R = 0..3; log-decays in
// base-2 units, gamma = clamp(g) * log2(e)):
//   L_r    inclusive cumulative gamma inside r's sub-tile;  tau_R its total
//   ref_R  sum of tau over earlier sub-tiles (chunk-relative start of R)
//   A[r,i] = beta_r sum_c k_rc k_ic 2^(G_rc - G_ic)     i < r   (G = ref + L)
//   P[r,i] =        sum_c q_rc k_ic 2^(G_rc - G_ic)     i <= r
//   T      = (I + A)^-1 Diag(beta)        (UT / WY form of the delta rule)
//   W      = T (k 2^G),   U0 = T V
//   U      = U0 - W S                     (S = state entering the chunk)
//   O      = (q 2^G) S + P U
//   S'     = Diag(2^G_end) S + (k 2^(G_end - G))^T U
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
// accumulation.  The output path through P (q 2^L, the column operand, P
// itself) and U are carried as hi + lo bfloat16 pairs (three products per
// pair of split operands); A, T, W, (q 2^G), S and the state-update key
// operand are single bfloat16.  float32 inputs use the float32 MFMA throughout.
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


constexpr int kC = 64;    // chunk
constexpr int kSub = 16;  // sub-tile
constexpr int kNSub = 4;

template <typename TIn, int DK, int DVS>
struct PrefillLayout {
  static constexpr bool BF16 = sizeof(TIn) == 2;
  typedef typename Mfma<BF16>::op_t op_t;
  static constexpr int OPB = sizeof(op_t);
  static constexpr int PAD = 16 / OPB;
  static constexpr int LDK = DK + PAD;  // [x][DK] operand arrays
  static constexpr int LDC = kC + PAD;  // [x][64] operand arrays (k = token)
  static constexpr int LDF = DK + 4;    // [64][DK] float32
  static constexpr int LDA = kC + 4;    // [64][64] float32

  static constexpr int SZ_K = kC * LDK * OPB;
  static constexpr int SZ_Q2 = BF16 ? kC * LDK * OPB : 0;
  static constexpr int SZ_L = kC * LDF * 4;
  static constexpr int SZ_KCT = DK * LDC * OPB;
  static constexpr int SZ_QC = kC * LDK * OPB;
  static constexpr int SZ_TF = kC * LDA * 4;
  static constexpr int SZ_TB = kC * LDC * OPB;
  static constexpr int SZ_UT = (BF16 ? 2 : 1) * DVS * LDC * OPB;
  static constexpr int PH1 = 2 * SZ_K + SZ_Q2 + SZ_L;
  static constexpr int PH2 = 2 * SZ_KCT + SZ_QC + SZ_TF + SZ_TB;
  static constexpr int REGION = PH1 > PH2 ? PH1 : PH2;
  // phase-1 view of the shared region
  static constexpr int O_K = 0, O_Q = SZ_K, O_Q2 = 2 * SZ_K, O_L = 2 * SZ_K + SZ_Q2;
  // phase-2 view: dead-first order so U^T can reuse KcT | Tf | Tb
  static constexpr int O_KCT = 0, O_TF = SZ_KCT, O_TB = SZ_KCT + SZ_TF;
  static constexpr int O_QC = O_TB + SZ_TB, O_KBT = O_QC + SZ_QC;
  static constexpr int O_UT = 0;
  static_assert(SZ_UT <= SZ_KCT + SZ_TF + SZ_TB, "U^T must fit in the dead prefix");
  // persistent / per-chunk buffers outside the region
  static constexpr int SZ_AW = (kC * LDA * 4 > kC * LDK * OPB) ? kC * LDA * 4 : kC * LDK * OPB;
  static constexpr int O_A = REGION;  // A, then W
  static constexpr int O_P = O_A + SZ_AW;
  static constexpr int O_VT = O_P + kC * LDA * 4;
  static constexpr int O_ST = O_VT + DVS * LDC * OPB;
  static constexpr int O_SM = O_ST + DVS * LDK * OPB;
  // small float32 arrays: beta[64], tau[4][DK], eref[4][DK], ebar[4][DK], pair[6][DK], egam[DK]
  static constexpr int SM_BETA = 0, SM_TAU = 64, SM_EREF = 64 + 4 * DK, SM_EBAR = 64 + 8 * DK;
  static constexpr int SM_PAIR = 64 + 12 * DK, SM_EGAM = 64 + 18 * DK;
  static constexpr int SZ_SM = (64 + 19 * DK) * 4;
  static constexpr int TOTAL = O_SM + SZ_SM;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

template <typename TIn, typename TOut, int DK, int DV, int DVS, int NW>
__global__ void __launch_bounds__(NW * 64) chunk_fwd_kernel(PrefillArgs p) {
  typedef PrefillLayout<TIn, DK, DVS> Lay;
  constexpr bool BF16 = Lay::BF16;
  typedef Mfma<BF16> M;
  typedef typename M::op_t op_t;
  typedef typename M::frag frag;
  constexpr int NT = NW * 64;
  constexpr int KS = M::KSTEP, KPL = M::KPL;
  constexpr int LDK = Lay::LDK, LDC = Lay::LDC, LDF = Lay::LDF, LDA = Lay::LDA;
  constexpr int NSLICE = DV / DVS;
  constexpr int NST = (DK / 16) * (DVS / 16);  // state tiles
  constexpr int NSW = NST / NW;
  constexpr int NU = (kC / 16) * (DVS / 16);  // U / O tiles
  constexpr int NUW = (NU + NW - 1) / NW;
  static_assert(NST % NW == 0, "state tiles per wave");
  static_assert(NW >= 4, "the sub-tile solve uses four waves");

  extern __shared__ __align__(16) unsigned char smem[];
  op_t* sK = reinterpret_cast<op_t*>(smem + Lay::O_K);
  op_t* sQ = reinterpret_cast<op_t*>(smem + Lay::O_Q);
  op_t* sQ2 = reinterpret_cast<op_t*>(smem + Lay::O_Q2);
  float* sL = reinterpret_cast<float*>(smem + Lay::O_L);
  op_t* sKcT = reinterpret_cast<op_t*>(smem + Lay::O_KCT);
  float* sTf = reinterpret_cast<float*>(smem + Lay::O_TF);
  op_t* sTb = reinterpret_cast<op_t*>(smem + Lay::O_TB);
  op_t* sQc = reinterpret_cast<op_t*>(smem + Lay::O_QC);
  op_t* sKbT = reinterpret_cast<op_t*>(smem + Lay::O_KBT);
  op_t* sUT = reinterpret_cast<op_t*>(smem + Lay::O_UT);
  op_t* sUT2 = sUT + DVS * LDC;  // lo part (bf16 only)
  float* sA = reinterpret_cast<float*>(smem + Lay::O_A);
  op_t* sW = reinterpret_cast<op_t*>(smem + Lay::O_A);
  float* sP = reinterpret_cast<float*>(smem + Lay::O_P);
  op_t* sVT = reinterpret_cast<op_t*>(smem + Lay::O_VT);
  op_t* sST = reinterpret_cast<op_t*>(smem + Lay::O_ST);
  float* sm = reinterpret_cast<float*>(smem + Lay::O_SM);
  float* sBeta = sm + Lay::SM_BETA;
  float* sTau = sm + Lay::SM_TAU;
  float* sERef = sm + Lay::SM_EREF;
  float* sEBar = sm + Lay::SM_EBAR;
  float* sPair = sm + Lay::SM_PAIR;
  float* sEGam = sm + Lay::SM_EGAM;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int kofs = lg * KPL;

  // Workgroup -> (head, slice): consecutive workgroups are dealt round-robin to
  // the 8 XCDs, so give all slices of a head the same XCD (and L2).
  const int64_t nheads = p.B * p.H;
  const int64_t x = blockIdx.x;
  const int64_t grp = x / (8 * NSLICE);
  const int gi = (int)(x % (8 * NSLICE));
  const int64_t head = grp * 8 + (gi % 8);
  const int slice = gi / 8;
  if (head >= nheads) return;
  const int64_t b = head / p.H, h = head % p.H;
  const int j0 = slice * DVS;
  const int64_t T = p.T, H = p.H;

  const TIn* gq = reinterpret_cast<const TIn*>(p.q);
  const TIn* gk = reinterpret_cast<const TIn*>(p.k);
  const TIn* gv = reinterpret_cast<const TIn*>(p.v);
  const TIn* gg = reinterpret_cast<const TIn*>(p.g);
  const TIn* gb = reinterpret_cast<const TIn*>(p.beta);
  TOut* go = reinterpret_cast<TOut*>(p.o);
  const int64_t state_off = head * (int64_t)DK * DV;

  // ---- state slice in accumulators (D layout: row 4*lg+m, col l16 of a 16x16 tile)
  f32x4 Sacc[NSW];
#pragma unroll
  for (int i = 0; i < NSW; ++i) {
    const int tt = wave + NW * i;
    const int ct = tt / (DVS / 16), jt = tt % (DVS / 16);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int c = 16 * ct + 4 * lg + m, jv = 16 * jt + l16;
      Sacc[i][m] = p.s0 ? p.s0[state_off + (int64_t)c * DV + j0 + jv] : 0.f;
    }
  }

  auto store_state_operand = [&]() {
#pragma unroll
    for (int i = 0; i < NSW; ++i) {
      const int tt = wave + NW * i;
      const int ct = tt / (DVS / 16), jt = tt % (DVS / 16);
      op_t* dst = sST + (16 * jt + l16) * LDK + 16 * ct + 4 * lg;
#pragma unroll
      for (int m = 0; m < 4; ++m) dst[m] = from_f32<op_t>(Sacc[i][m]);
    }
  };
  store_state_operand();

  const int64_t nchunks = (T + kC - 1) / kC;
  constexpr int E16 = 16 / sizeof(TIn);  // input elements per 16-byte load
  constexpr int CGP = DK / 8;            // prep: groups of 8 channels
  constexpr int RP = NT / CGP;           // prep: rows per pass
  constexpr int NP = kC / RP;            // prep: passes
  static_assert(NP * RP == kC, "prep layout");

  for (int64_t n = 0; n < nchunks; ++n) {
    const int64_t t0 = n * kC;
    // ---- step 0: stage the chunk (k, q raw; g -> gamma; v^T; beta)
    for (int pc = tid; pc < kC * DK / E16; pc += NT) {
      const int r = pc / (DK / E16), c = (pc % (DK / E16)) * E16;
      const int64_t t = t0 + r;
      float gf[E16];
      if (t < T) {
        const int64_t off = ((b * T + t) * H + h) * DK + c;
        *reinterpret_cast<float4*>(sK + r * LDK + c) = *reinterpret_cast<const float4*>(gk + off);
        *reinterpret_cast<float4*>(sQ + r * LDK + c) = *reinterpret_cast<const float4*>(gq + off);
        load16(gg + off, gf);
#pragma unroll
        for (int e = 0; e < E16; ++e) gf[e] = clamp_log_decay(gf[e]) * kLog2e;
      } else {
        *reinterpret_cast<float4*>(sK + r * LDK + c) = make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(sQ + r * LDK + c) = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int e = 0; e < E16; ++e) gf[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < E16; ++e) sL[r * LDF + c + e] = gf[e];
    }
    for (int pc = tid; pc < kC * DVS / E16; pc += NT) {
      const int r = pc / (DVS / E16), jv = (pc % (DVS / E16)) * E16;
      const int64_t t = t0 + r;
      float vf[E16];
      if (t < T) {
        load16(gv + ((b * T + t) * H + h) * DV + j0 + jv, vf);
      } else {
#pragma unroll
        for (int e = 0; e < E16; ++e) vf[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < E16; ++e) sVT[(jv + e) * LDC + r] = from_f32<op_t>(vf[e]);
    }
    if (tid < kC) {
      const int64_t t = t0 + tid;
      sBeta[tid] = (t < T) ? to_f32(gb[(b * T + t) * H + h]) : 0.f;
    }
    __syncthreads();

    // ---- step 1: sub-tile cumulative log-decay and per-(sub-tile, channel) factors
    for (int pr = tid; pr < kNSub * DK; pr += NT) {
      const int c = pr % DK, R = pr / DK;
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < kSub; ++j) {
        float* e = sL + (kSub * R + j) * LDF + c;
        acc += *e;
        *e = acc;
      }
      sTau[R * DK + c] = acc;
    }
    __syncthreads();
    for (int c = tid; c < DK; c += NT) {
      const float t0_ = sTau[c], t1 = sTau[DK + c], t2 = sTau[2 * DK + c], t3 = sTau[3 * DK + c];
      sERef[c] = 1.f;
      sERef[DK + c] = exp2_hw(t0_);
      sERef[2 * DK + c] = exp2_hw(t0_ + t1);
      sERef[3 * DK + c] = exp2_hw(t0_ + t1 + t2);
      sEBar[3 * DK + c] = exp2_hw(t3);
      sEBar[2 * DK + c] = exp2_hw(t2 + t3);
      sEBar[DK + c] = exp2_hw(t1 + t2 + t3);
      sEBar[c] = exp2_hw(t0_ + t1 + t2 + t3);
      sEGam[c] = exp2_hw(t0_ + t1 + t2 + t3);
      // pair (R, I < R) -> index R(R-1)/2 + I, factor 2^(sum_{J=I}^{R-1} tau_J)
      sPair[0 * DK + c] = exp2_hw(t0_);            // (1,0)
      sPair[1 * DK + c] = exp2_hw(t0_ + t1);       // (2,0)
      sPair[2 * DK + c] = exp2_hw(t1);             // (2,1)
      sPair[3 * DK + c] = exp2_hw(t0_ + t1 + t2);  // (3,0)
      sPair[4 * DK + c] = exp2_hw(t1 + t2);        // (3,1)
      sPair[5 * DK + c] = exp2_hw(t2);             // (3,2)
    }
    __syncthreads();

    // ---- step 2: operands. In place: k -> k 2^L, q -> q 2^L (hi), L -> k 2^-L.
    // The chunk-relative operands are kept in registers until the A/P products
    // have released the shared region.
    typedef op_t vec8 __attribute__((ext_vector_type(8)));
    vec8 dKc[NP], dQc[NP], dKb[NP];
#pragma unroll
    for (int mm = 0; mm < NP; ++mm) {
      const int r = tid / CGP + RP * mm, c0 = 8 * (tid % CGP), R = r / kSub;
      float kf[8], qf[8], lf[8];
      load8(sK + r * LDK + c0, kf);
      load8(sQ + r * LDK + c0, qf);
      load8(sL + r * LDF + c0, lf);
      vec8 vkr, vqh, vql;
      float kd[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ep = exp2_hw(lf[e]), em = exp2_hw(-lf[e]);
        const float kr = kf[e] * ep, qr = qf[e] * ep;
        kd[e] = kf[e] * em;
        vkr[e] = from_f32<op_t>(kr);
        vqh[e] = from_f32<op_t>(qr);
        vql[e] = from_f32<op_t>(qr - to_f32(vqh[e]));
        const float er = sERef[R * DK + c0 + e], eb = sEBar[R * DK + c0 + e];
        dKc[mm][e] = from_f32<op_t>(kr * er);
        dQc[mm][e] = from_f32<op_t>(qr * er);
        dKb[mm][e] = from_f32<op_t>(kd[e] * eb);
      }
      *reinterpret_cast<vec8*>(sK + r * LDK + c0) = vkr;
      *reinterpret_cast<vec8*>(sQ + r * LDK + c0) = vqh;
      if constexpr (BF16) *reinterpret_cast<vec8*>(sQ2 + r * LDK + c0) = vql;
      store8(sL + r * LDF + c0, kd);
    }
    __syncthreads();

    // ---- step 3: A and P tiles, every tile pair one dense product
    for (int pi = wave; pi < 10; pi += NW) {
      // pair order (R, I): (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3)
      const int R = pi < 1 ? 0 : pi < 3 ? 1 : pi < 6 ? 2 : 3;
      const int I = pi - R * (R + 1) / 2;
      const float* pair = (I < R) ? sPair + (R * (R - 1) / 2 + I) * DK : nullptr;
      f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
      const int row = kSub * R + l16, col = kSub * I + l16;
#pragma unroll 2
      for (int kk = 0; kk < DK; kk += KS) {
        const int k0 = kk + kofs;
        const frag aK = M::ld(sK + row * LDK + k0);
        const frag aQ = M::ld(sQ + row * LDK + k0);
        if constexpr (BF16) {
          const frag aQ2 = M::ld(sQ2 + row * LDK + k0);
          float cf[8];
          load8(sL + col * LDF + k0, cf);
          if (pair) {
            float pf[8];
            load8(pair + k0, pf);
#pragma unroll
            for (int e = 0; e < 8; ++e) cf[e] *= pf[e];
          }
          frag bh, bl;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const __bf16 hh = (__bf16)cf[e];
            bh[e] = hh;
            bl[e] = (__bf16)(cf[e] - (float)hh);
          }
          accA = M::mma(aK, bh, accA);
          accP = M::mma(aQ, bh, accP);
          accP = M::mma(aQ2, bh, accP);
          accP = M::mma(aQ, bl, accP);
        } else {
          float cf = sL[col * LDF + k0];
          if (pair) cf *= pair[k0];
          accA = M::mma(aK, cf, accA);
          accP = M::mma(aQ, cf, accP);
        }
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = kSub * R + 4 * lg + m, i = col;
        sA[r * LDA + i] = (i < r) ? sBeta[r] * accA[m] : 0.f;
        sP[r * LDA + i] = (i <= r) ? accP[m] : 0.f;
      }
    }
    // zero the tiles above the diagonal
    for (int e = tid; e < 6 * 256; e += NT) {
      const int u = e / 256, w = e % 256;
      const int R = u < 3 ? 0 : u < 5 ? 1 : 2;
      const int I = u < 3 ? u + 1 : u < 5 ? u - 1 : 3;
      const int r = kSub * R + w / 16, i = kSub * I + w % 16;
      sA[r * LDA + i] = 0.f;
      sP[r * LDA + i] = 0.f;
    }
    __syncthreads();

    // deferred operands into the released region
#pragma unroll
    for (int mm = 0; mm < NP; ++mm) {
      const int r = tid / CGP + RP * mm, c0 = 8 * (tid % CGP);
      *reinterpret_cast<vec8*>(sQc + r * LDK + c0) = dQc[mm];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sKcT[(c0 + e) * LDC + r] = dKc[mm][e];
        sKbT[(c0 + e) * LDC + r] = dKb[mm][e];
      }
    }

    // ---- step 4: T = (I + A)^-1 (float32).  4a: the four 16x16 diagonal blocks
    if (wave < 4) {
      const int R = wave;
      float X[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) X[m] = (4 * lg + m == l16) ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < kSub - 1; ++i) {
        const float xi = __shfl(X[i & 3], l16 + 16 * (i >> 2), 64);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int r = 4 * lg + m;
          if (r > i) X[m] -= sA[(kSub * R + r) * LDA + kSub * R + i] * xi;
        }
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = kSub * R + 4 * lg + m;
        sTf[r * LDA + kSub * R + l16] = X[m];
      }
    }
    for (int e = tid; e < 6 * 256; e += NT) {  // zero the blocks above the diagonal
      const int u = e / 256, w = e % 256;
      const int R = u < 3 ? 0 : u < 5 ? 1 : 2;
      const int I = u < 3 ? u + 1 : u < 5 ? u - 1 : 3;
      sTf[(kSub * R + w / 16) * LDA + kSub * I + w % 16] = 0.f;
    }
    __syncthreads();
    // 4b: block rows R = 1..3: T_RI = -T_RR sum_{J=I}^{R-1} A_RJ T_JI
    float* sY = reinterpret_cast<float*>(sTb);  // 16x16 float32 scratch per wave
#pragma unroll
    for (int R = 1; R < kNSub; ++R) {
      if (wave < R) {
        const int I = wave;
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        for (int j = kSub * I; j < kSub * R; j += 4) {
          const float a = sA[(kSub * R + l16) * LDA + j + lg];
          const float bb = sTf[(j + lg) * LDA + kSub * I + l16];
          y = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, y, 0, 0, 0);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) sY[wave * 256 + (4 * lg + m) * 16 + l16] = y[m];
      }
      __syncthreads();
      if (wave < R) {
        const int I = wave;
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kSub; j += 4) {
          const float a = sTf[(kSub * R + l16) * LDA + kSub * R + j + lg];
          const float bb = sY[wave * 256 + (j + lg) * 16 + l16];
          t = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, t, 0, 0, 0);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m)
          sTf[(kSub * R + 4 * lg + m) * LDA + kSub * I + l16] = -t[m];
      }
      __syncthreads();
    }
    // 4c: T' = T Diag(beta) as an MFMA operand
    for (int e = tid; e < kC * kC; e += NT) {
      const int r = e / kC, j = e % kC;
      sTb[r * LDC + j] = from_f32<op_t>(sTf[r * LDA + j] * sBeta[j]);
    }
    __syncthreads();

    // ---- step 5: W = T' Kc  (-> shared, A's slot), U0 = T' V (-> registers)
    for (int tt = wave; tt < 4 * (DK / 16); tt += NW) {
      const int rt = tt / (DK / 16), ct = tt % (DK / 16);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kC; kk += KS) {
        acc = M::mma(M::ld(sTb + (16 * rt + l16) * LDC + kk + kofs),
                     M::ld(sKcT + (16 * ct + l16) * LDC + kk + kofs), acc);
      }
#pragma unroll
      for (int m = 0; m < 4; ++m)
        sW[(16 * rt + 4 * lg + m) * LDK + 16 * ct + l16] = from_f32<op_t>(acc[m]);
    }
    f32x4 Uacc[NUW];
#pragma unroll
    for (int i = 0; i < NUW; ++i) {
      const int tt = wave + NW * i;
      Uacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (tt < NU) {
        const int rt = tt / (DVS / 16), jt = tt % (DVS / 16);
#pragma unroll
        for (int kk = 0; kk < kC; kk += KS) {
          Uacc[i] = M::mma(M::ld(sTb + (16 * rt + l16) * LDC + kk + kofs),
                           M::ld(sVT + (16 * jt + l16) * LDC + kk + kofs), Uacc[i]);
        }
      }
    }
    __syncthreads();

    // ---- step 6: U = U0 - W S  -> U^T (hi/lo) in shared
#pragma unroll
    for (int i = 0; i < NUW; ++i) {
      const int tt = wave + NW * i;
      if (tt < NU) {
        const int rt = tt / (DVS / 16), jt = tt % (DVS / 16);
        f32x4 ws = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int kk = 0; kk < DK; kk += KS) {
          ws = M::mma(M::ld(sW + (16 * rt + l16) * LDK + kk + kofs),
                      M::ld(sST + (16 * jt + l16) * LDK + kk + kofs), ws);
        }
        const int jv = 16 * jt + l16, i0 = 16 * rt + 4 * lg;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float u = Uacc[i][m] - ws[m];
          const op_t uh = from_f32<op_t>(u);
          sUT[jv * LDC + i0 + m] = uh;
          if constexpr (BF16) sUT2[jv * LDC + i0 + m] = from_f32<op_t>(u - to_f32(uh));
        }
      }
    }
    __syncthreads();

    // ---- step 7: O = Qc S + P U
#pragma unroll
    for (int i = 0; i < NUW; ++i) {
      const int tt = wave + NW * i;
      if (tt < NU) {
        const int rt = tt / (DVS / 16), jt = tt % (DVS / 16);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int kk = 0; kk < DK; kk += KS) {
          acc = M::mma(M::ld(sQc + (16 * rt + l16) * LDK + kk + kofs),
                       M::ld(sST + (16 * jt + l16) * LDK + kk + kofs), acc);
        }
        const int kend = 16 * rt + 16;  // P is lower triangular
        for (int kk = 0; kk < kend; kk += KS) {
          const int k0 = kk + kofs;
          if constexpr (BF16) {
            float pf[8];
            load8(sP + (16 * rt + l16) * LDA + k0, pf);
            frag ph, pl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const __bf16 hh = (__bf16)pf[e];
              ph[e] = hh;
              pl[e] = (__bf16)(pf[e] - (float)hh);
            }
            const frag uh = M::ld(sUT + (16 * jt + l16) * LDC + k0);
            const frag ul = M::ld(sUT2 + (16 * jt + l16) * LDC + k0);
            acc = M::mma(ph, uh, acc);
            acc = M::mma(pl, uh, acc);
            acc = M::mma(ph, ul, acc);
          } else {
            acc = M::mma(sP[(16 * rt + l16) * LDA + k0], sUT[(16 * jt + l16) * LDC + k0], acc);
          }
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int64_t t = t0 + 16 * rt + 4 * lg + m;
          if (t < T) go[((b * T + t) * H + h) * DV + j0 + 16 * jt + l16] = from_f32<TOut>(acc[m]);
        }
      }
    }

    // ---- step 8: S <- Diag(2^G_end) S + Kbar^T U
#pragma unroll
    for (int i = 0; i < NSW; ++i) {
      const int tt = wave + NW * i;
      const int ct = tt / (DVS / 16), jt = tt % (DVS / 16);
#pragma unroll
      for (int m = 0; m < 4; ++m) Sacc[i][m] *= sEGam[16 * ct + 4 * lg + m];
#pragma unroll
      for (int kk = 0; kk < kC; kk += KS) {
        const frag a = M::ld(sKbT + (16 * ct + l16) * LDC + kk + kofs);
        Sacc[i] = M::mma(a, M::ld(sUT + (16 * jt + l16) * LDC + kk + kofs), Sacc[i]);
        if constexpr (BF16) Sacc[i] = M::mma(a, M::ld(sUT2 + (16 * jt + l16) * LDC + kk + kofs), Sacc[i]);
      }
    }
    __syncthreads();
    store_state_operand();

    if (p.ck && ((n + 1) * kC) % p.ck_every == 0 && (n + 1) * kC <= T) {
      const int64_t nck = T / p.ck_every, idx = (n + 1) * kC / p.ck_every - 1;
      float* dst = p.ck + ((b * nck + idx) * H + h) * (int64_t)DK * DV;
#pragma unroll
      for (int i = 0; i < NSW; ++i) {
        const int tt = wave + NW * i;
        const int ct = tt / (DVS / 16), jt = tt % (DVS / 16);
#pragma unroll
        for (int m = 0; m < 4; ++m)
          dst[(int64_t)(16 * ct + 4 * lg + m) * DV + j0 + 16 * jt + l16] = Sacc[i][m];
      }
    }
  }

  if (p.s_final) {
#pragma unroll
    for (int i = 0; i < NSW; ++i) {
      const int tt = wave + NW * i;
      const int ct = tt / (DVS / 16), jt = tt % (DVS / 16);
#pragma unroll
      for (int m = 0; m < 4; ++m)
        p.s_final[state_off + (int64_t)(16 * ct + 4 * lg + m) * DV + j0 + 16 * jt + l16] =
            Sacc[i][m];
    }
  }
}

template <typename TIn, typename TOut, int DK, int DV, int DVS, int NW>
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  typedef PrefillLayout<TIn, DK, DVS> Lay;
  auto kern = chunk_fwd_kernel<TIn, TOut, DK, DV, DVS, NW>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     Lay::TOTAL);
  if (e != hipSuccess) return e;
  constexpr int NSLICE = DV / DVS;
  const int64_t nheads = a.B * a.H;
  const int64_t groups = (nheads + 7) / 8;
  const int64_t grid = groups * 8 * NSLICE;
  kern<<<dim3((unsigned)grid), dim3(NW * 64), Lay::TOTAL, stream>>>(a);
  return hipGetLastError();
}

// d_v slice width per workgroup (must match the instantiations in chunk_fwd).
static int prefill_slice(int dk, int dv, bool in_bf16) {
  if (!in_bf16) return 64;
  return dk == 128 ? 64 : 32;
}

int64_t prefill_grid(int64_t heads, int dk, int dv, bool in_bf16) {
  return ((heads + 7) / 8) * 8 * (dv / prefill_slice(dk, dv, in_bf16));
}

hipError_t chunk_fwd(const PrefillArgs& a, int dk, int dv, bool in_bf16, bool out_bf16,
                     hipStream_t s) {
  if (in_bf16) {
    if (out_bf16) {
      if (dk == 128 && dv == 128) return launch_prefill<__bf16, __bf16, 128, 128, 64, 4>(a, s);
      if (dk == 128 && dv == 64) return launch_prefill<__bf16, __bf16, 128, 64, 64, 4>(a, s);
      if (dk == 64 && dv == 128) return launch_prefill<__bf16, __bf16, 64, 128, 32, 4>(a, s);
      return launch_prefill<__bf16, __bf16, 64, 64, 32, 4>(a, s);
    }
    if (dk == 128 && dv == 128) return launch_prefill<__bf16, float, 128, 128, 64, 4>(a, s);
    if (dk == 128 && dv == 64) return launch_prefill<__bf16, float, 128, 64, 64, 4>(a, s);
    if (dk == 64 && dv == 128) return launch_prefill<__bf16, float, 64, 128, 32, 4>(a, s);
    return launch_prefill<__bf16, float, 64, 64, 32, 4>(a, s);
  }
  if (out_bf16) return launch_prefill<float, __bf16, 64, 64, 64, 4>(a, s);
  return launch_prefill<float, float, 64, 64, 64, 4>(a, s);
}

}  // namespace kda
