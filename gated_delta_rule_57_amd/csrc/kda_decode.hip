// Single-token KDA recurrent update (decode), one workgroup per (sequence, head).
//
// Per (n, h), with S the d_k x d_v float32 state (rows = key channels):
//   S' = Diag(exp g') S,  a = S'^T k,  b = S'^T q,  u = beta (v - a),
//   S  <- S' + k u^T,     o = b + (k . q) u          (= S^T q after the write)
// which is the delta-rule step with KDA's per-channel decay (Towards-AI article
// on Kimi K3, "Kimi Delta Attention (KDA)"), updated in place as the orkas.ai
// blog's "The cost is paid in the serving stack" section describes for decoding.
//
// The step is bound by HBM: the 64 KiB state of a head is read once and
// written once.  Each of the 256 threads keeps RPT rows x 4 columns of the
// state in registers between the read and the write, loaded and stored with
// 128-bit accesses; consecutive lanes cover consecutive 16-byte pieces of a
// row, so a wavefront touches 1 KiB of contiguous state per access.  The two
// column reductions (a and b) go through LDS once.
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <typename TIn, typename TOut, int DK, int DV, bool LOGITS>
__global__ void __launch_bounds__(256) decode_step_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const TIn* __restrict__ g, const TIn* __restrict__ beta, float* __restrict__ state,
    TOut* __restrict__ o, int64_t n_heads_total, const TIn* __restrict__ ogate) {
  constexpr int NT = 256;
  constexpr int CG = DV / 4;    // column groups of 4 floats
  constexpr int RG = NT / CG;   // row groups
  constexpr int RPT = DK / RG;  // rows per thread
  static_assert(RPT * RG == DK && CG * RG == NT, "thread layout");

  const int64_t hd = blockIdx.x;
  if (hd >= n_heads_total) return;
  const int t = threadIdx.x;
  const int cg = t % CG;
  const int rg = t / CG;

  __shared__ float s_q[DK], s_k[DK], s_dec[DK];
  __shared__ float s_part_a[RG][DV], s_part_b[RG][DV];
  __shared__ float s_u[DV];
  __shared__ float s_kq;

  float4* st = reinterpret_cast<float4*>(state + hd * (int64_t)(DK * DV));
  float4 S[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) S[i] = st[(rg + RG * i) * CG + cg];

  if (t < DK) {
    const int64_t off = hd * DK + t;
    s_q[t] = to_f32(q[off]);
    s_k[t] = to_f32(k[off]);
    s_dec[t] = exp2_hw(LOGITS ? gamma_from_logit(to_f32(g[off]))
                              : clamp_log_decay(to_f32(g[off])) * kLog2e);
  }
  __syncthreads();
  if (t < 64) {
    float x = 0.f;
#pragma unroll
    for (int c = t; c < DK; c += 64) x += s_q[c] * s_k[c];
    x = wave_sum(x);
    if (t == 0) s_kq = x;
  }

  float4 pa = {0.f, 0.f, 0.f, 0.f}, pb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int c = rg + RG * i;
    const float d = s_dec[c], kc = s_k[c], qc = s_q[c];
    S[i].x *= d;
    S[i].y *= d;
    S[i].z *= d;
    S[i].w *= d;
    pa.x += kc * S[i].x;
    pa.y += kc * S[i].y;
    pa.z += kc * S[i].z;
    pa.w += kc * S[i].w;
    pb.x += qc * S[i].x;
    pb.y += qc * S[i].y;
    pb.z += qc * S[i].z;
    pb.w += qc * S[i].w;
  }
  *reinterpret_cast<float4*>(&s_part_a[rg][4 * cg]) = pa;
  *reinterpret_cast<float4*>(&s_part_b[rg][4 * cg]) = pb;
  __syncthreads();

  if (t < DV) {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      a += s_part_a[r][t];
      b += s_part_b[r][t];
    }
    const float bt = to_f32(beta[hd]);
    const float u = bt * (to_f32(v[hd * DV + t]) - a);
    s_u[t] = u;
    float ov = b + s_kq * u;
    if (ogate) ov *= sigmoid_hw(to_f32(ogate[hd * DV + t]));  // output gate, if given
    o[hd * DV + t] = from_f32<TOut>(ov);
  }
  __syncthreads();

  const float4 u4 = *reinterpret_cast<const float4*>(&s_u[4 * cg]);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int c = rg + RG * i;
    const float kc = s_k[c];
    float4 x = S[i];
    x.x += kc * u4.x;
    x.y += kc * u4.y;
    x.z += kc * u4.z;
    x.w += kc * u4.w;
    // The state is not read again by this launch: a streaming store keeps it
    // from displacing lines that other workgroups are still reading.
    __builtin_nontemporal_store(f32x4{x.x, x.y, x.z, x.w},
                                reinterpret_cast<f32x4*>(&st[c * CG + cg]));
  }
}

// Speculative decoding: K draft tokens per sequence, inputs [N, K, H, .].
//   VERIFY: o for every draft token from the committed state; the state is read only.
//   COMMIT: the state of sequence n advanced in place by accept[n] tokens (clamped
//           to [0, K]); q and o unused.
// The draft tokens' projected inputs are all that is kept; the state of an
// accepted prefix is rebuilt on chip from them (the orkas.ai blog "Kimi K3
// architecture", section "The cost is paid in the serving stack", describes
// this in place of rolling back an in-place update).
//
// A workgroup keeps one (sequence, head) state slice in registers (as the
// single-token kernel does) across the tokens.  The inputs of up to KB tokens are
// loaded into shared memory at once (with the cumulative decays and k.q computed
// there), so the token loop has no global loads and two barriers per token.
// 512 threads (eight waves) keep RPT = 8 or fewer state rows x 4 columns per
// thread.  256-thread workgroups (twice the values per thread, fewer waves)
// measured 5-7% slower; 1024 no faster for a commit and far slower for a
// verification.
//
// A verification only reads the state.  It loads it after the first block's own
// inputs, so that staging the inputs and their decays need not wait for the 64 KiB
// of state (loads retire in order), and with streaming loads, which keep it out of
// the caches (-8% time together).  Asking for six waves per SIMD keeps it at 80
// VGPRs, three workgroups per CU instead of two.  A commit writes its state back;
// the same load order and streaming loads measured slower for it (and for the
// single-token step), so it loads its state first, and fits eight waves per SIMD
// without asking.
constexpr int kMultiThreads = 512;

// A global-memory pointer that is the same in every lane, held in scalar
// registers (so that a lane adds only a 32-bit offset to it).
typedef const char __attribute__((address_space(1)))* global_cptr;
__device__ __forceinline__ global_cptr uniform_ptr(const char* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (global_cptr)(((uint64_t)hi << 32) | lo);
}

template <typename TIn, typename TOut, int DK, int DV, bool COMMIT>
__global__ void __launch_bounds__(kMultiThreads) __attribute__((amdgpu_waves_per_eu(COMMIT ? 1 : 6)))
multi_token_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const TIn* __restrict__ g, const TIn* __restrict__ beta, const int32_t* __restrict__ accept,
    float* __restrict__ state, TOut* __restrict__ o, int64_t N, int64_t K, int64_t H) {
  constexpr int NT = kMultiThreads, KB = 8;
  constexpr int CG = DV / 4, RG = NT / CG, RPT = DK / RG;
  // element pairs of one block's [KB][DK] and [KB][DV] inputs per thread
  constexpr int EP = (KB * DK / 2 + NT - 1) / NT, EQ = (KB * DV / 2 + NT - 1) / NT;
  static_assert(RPT * RG == DK && CG * RG == NT, "thread layout");
  constexpr bool WANT_O = !COMMIT;
  const int64_t hd = blockIdx.x;  // n * H + h
  if (hd >= N * H) return;
  const int64_t n = hd / H, h = hd % H;
  int64_t steps = K;
  if (COMMIT) {
    const int64_t a = accept[n];
    steps = a < 0 ? 0 : (a > K ? K : a);
    if (steps == 0) return;
  }
  // Inside a block the state is carried undecayed, S~ = Diag(Gamma_j)^-1 S with Gamma_j
  // the block's cumulative decay through token j: the decay moves from every state
  // element onto the token's key and query vectors (k Gamma_j, q Gamma_j, k / Gamma_j),
  // and the state is decayed once at the end of the block.  Gamma_j >= 2^(-5 log2e KB),
  // so 1 / Gamma_j stays a normal float.
  __shared__ float s_qg[WANT_O ? KB : 1][DK], s_kg[KB][DK], s_ki[KB][DK], s_v[KB][DV];
  // (for a verification, s_beta has a slot per thread: stored without a branch)
  __shared__ float s_ge[DK], s_beta[WANT_O ? NT : KB], s_kq[KB];
  __shared__ float s_part_a[RG][DV], s_part_b[WANT_O ? RG : 1][DV];
  __shared__ float s_u[DV];

  const int t = threadIdx.x, cg = t % CG, rg = t / CG;
  auto load_state = [&](float4 (&X)[RPT], int64_t head) {
    if constexpr (COMMIT) {
      const float4* st = reinterpret_cast<const float4*>(state + head * (int64_t)(DK * DV));
#pragma unroll
      for (int i = 0; i < RPT; ++i) X[i] = st[(rg + RG * i) * CG + cg];
      return;
    }
    // a uniform 64-bit base and one 32-bit lane offset: rows step by a constant
    const char* src = reinterpret_cast<const char*>(state + head * (int64_t)(DK * DV));
    const uint32_t lane_off = (uint32_t)(rg * CG + cg) * 16u;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      typedef const f32x4 __attribute__((address_space(1)))* gf4;
      const gf4 p = (gf4)(uniform_ptr(src + (size_t)i * (RG * CG * 16)) + lane_off);
      const f32x4 x = __builtin_nontemporal_load(p);
      X[i] = float4{x[0], x[1], x[2], x[3]};
    }
  };
  float4 S[RPT];
  if (COMMIT) load_state(S, hd);

  // One block of up to KB tokens; a verification's first block is its own copy, so
  // that its state loads sit in straight-line code behind the inputs.
  auto block = [&](int64_t j0, auto first) {
    constexpr bool FIRST = decltype(first)::value;
    const int nb = (int)((steps - j0) < KB ? (steps - j0) : KB);
    if (!FIRST && j0 > 0) __syncthreads();  // the previous block is done with the inputs
    // this block's inputs (token j of the draft is [n, j, h]), raw: k, g (in the slot
    // of k / Gamma), q, v, beta
    if constexpr (COMMIT) {
      for (int e = t; e < nb * DK; e += NT) {
        const int j = e / DK, c = e % DK;
        const int64_t off = ((n * K + j0 + j) * H + h) * DK + c;
        s_kg[j][c] = to_f32(k[off]);
        s_ki[j][c] = to_f32(g[off]);
      }
      for (int e = t; e < nb * DV; e += NT) {
        const int j = e / DV, c = e % DV;
        s_v[j][c] = to_f32(v[((n * K + j0 + j) * H + h) * DV + c]);
      }
      if (t < nb) s_beta[t] = to_f32(beta[(n * K + j0 + t) * H + h]);
    } else {
      // Loaded into registers first, two consecutive elements per thread and load,
      // so that the state loads queue behind them; a token past the block's end
      // loads the block's last token (in bounds) into a row that is never read,
      // which keeps loads and stores free of branches
      typedef TIn pair_t __attribute__((ext_vector_type(2)));
      float xk[EP][2], xg[EP][2], xq[EP][2], xv[EQ][2];
#pragma unroll
      for (int i = 0; i < EP; ++i) {
        const int e = 2 * (t + NT * i);
        const int j = min(e / DK, nb - 1), c = e % DK;  // (in bounds for any e)
        const int64_t off = ((n * K + j0 + j) * H + h) * DK + c;
        const pair_t a = *reinterpret_cast<const pair_t*>(&q[off]);
        const pair_t b = *reinterpret_cast<const pair_t*>(&k[off]);
        const pair_t d = *reinterpret_cast<const pair_t*>(&g[off]);
        xq[i][0] = to_f32(a[0]), xq[i][1] = to_f32(a[1]);
        xk[i][0] = to_f32(b[0]), xk[i][1] = to_f32(b[1]);
        xg[i][0] = to_f32(d[0]), xg[i][1] = to_f32(d[1]);
      }
#pragma unroll
      for (int i = 0; i < EQ; ++i) {
        const int e = 2 * (t + NT * i);
        const int j = min(e / DV, nb - 1), c = e % DV;
        const pair_t a = *reinterpret_cast<const pair_t*>(&v[((n * K + j0 + j) * H + h) * DV + c]);
        xv[i][0] = to_f32(a[0]), xv[i][1] = to_f32(a[1]);
      }
      const float xb = to_f32(beta[(n * K + j0 + min(t, nb - 1)) * H + h]);
      if (FIRST) load_state(S, hd);  // (a verification's; a commit's are issued above)
#pragma unroll
      for (int i = 0; i < EP; ++i) {
        const int e = 2 * (t + NT * i);
        if (KB * DK / 2 % NT == 0 || e < KB * DK) {
          const int j = e / DK, c = e % DK;
          s_qg[j][c] = xq[i][0], s_qg[j][c + 1] = xq[i][1];
          s_kg[j][c] = xk[i][0], s_kg[j][c + 1] = xk[i][1];
          s_ki[j][c] = xg[i][0], s_ki[j][c + 1] = xg[i][1];
        }
      }
#pragma unroll
      for (int i = 0; i < EQ; ++i) {
        const int e = 2 * (t + NT * i);
        if (KB * DV / 2 % NT == 0 || e < KB * DV)
          s_v[e / DV][e % DV] = xv[i][0], s_v[e / DV][e % DV + 1] = xv[i][1];
      }
      s_beta[t] = xb;  // slots past the block's tokens are never read
    }
    __syncthreads();
    if (t < DK) {  // one thread per key channel: the cumulative decay over the block
      const int c = t;
      float G = 1.f;
      for (int j = 0; j < nb; ++j) {
        G *= exp2_hw(clamp_log_decay(s_ki[j][c]) * kLog2e);
        const float kk = s_kg[j][c];
        s_kg[j][c] = kk * G;
        s_ki[j][c] = kk * __builtin_amdgcn_rcpf(G);
        if (WANT_O) s_qg[j][c] *= G;
      }
      s_ge[c] = G;
    }
    __syncthreads();
    if (WANT_O) {  // k . q of each token (= (q Gamma) . (k / Gamma)): one wave per token
      const int w = t >> 6, l = t & 63;
      for (int j = w; j < nb; j += NT / 64) {
        float x = 0.f;
#pragma unroll
        for (int c = l; c < DK; c += 64) x += s_qg[j][c] * s_ki[j][c];
        x = wave_sum(x);
        if (l == 0) s_kq[j] = x;
      }
    }

    for (int j = 0; j < nb; ++j) {
      float4 pa = {0.f, 0.f, 0.f, 0.f}, pb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int c = rg + RG * i;
        const float kc = s_kg[j][c];
        pa.x += kc * S[i].x;
        pa.y += kc * S[i].y;
        pa.z += kc * S[i].z;
        pa.w += kc * S[i].w;
        if (WANT_O) {
          const float qc = s_qg[j][c];
          pb.x += qc * S[i].x;
          pb.y += qc * S[i].y;
          pb.z += qc * S[i].z;
          pb.w += qc * S[i].w;
        }
      }
      *reinterpret_cast<float4*>(&s_part_a[rg][4 * cg]) = pa;
      if (WANT_O) *reinterpret_cast<float4*>(&s_part_b[rg][4 * cg]) = pb;
      __syncthreads();
      if (t < DV) {
        float a = 0.f, bsum = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          a += s_part_a[r][t];
          if (WANT_O) bsum += s_part_b[r][t];
        }
        const float u = s_beta[j] * (s_v[j][t] - a);
        s_u[t] = u;
        if (WANT_O) o[((n * K + j0 + j) * H + h) * DV + t] = from_f32<TOut>(bsum + s_kq[j] * u);
      }
      __syncthreads();
      const float4 u4 = *reinterpret_cast<const float4*>(&s_u[4 * cg]);
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float kc = s_ki[j][rg + RG * i];
        S[i].x += kc * u4.x;
        S[i].y += kc * u4.y;
        S[i].z += kc * u4.z;
        S[i].w += kc * u4.w;
      }
      // the next token's partial sums overwrite s_part_* only after everyone has
      // read them (they were read before the barrier above); s_u is rewritten after
      // the next token's first barrier, by which time this update is done
    }
    if (COMMIT || j0 + KB < steps) {  // back to the decayed state: S = Diag(Gamma_last) S~
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float ge = s_ge[rg + RG * i];
        S[i].x *= ge;
        S[i].y *= ge;
        S[i].z *= ge;
        S[i].w *= ge;
      }
    }
  };
  if constexpr (COMMIT) {
    for (int64_t j0 = 0; j0 < steps; j0 += KB) block(j0, std::false_type{});
  } else {
    block(int64_t(0), std::true_type{});
    for (int64_t j0 = KB; j0 < steps; j0 += KB) block(j0, std::false_type{});
  }
  if (COMMIT) {
    f32x4* dst = reinterpret_cast<f32x4*>(state + hd * (int64_t)(DK * DV));
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      __builtin_nontemporal_store(f32x4{S[i].x, S[i].y, S[i].z, S[i].w},
                                  &dst[(rg + RG * i) * CG + cg]);
  }
}

template <typename TIn, typename TOut, int DK, int DV, bool LOGITS>
hipError_t launch_decode(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, float* state, void* o, int64_t nh,
                         const void* ogate, hipStream_t stream) {
  decode_step_kernel<TIn, TOut, DK, DV, LOGITS><<<dim3((unsigned)nh), dim3(256), 0, stream>>>(
      (const TIn*)q, (const TIn*)k, (const TIn*)v, (const TIn*)g, (const TIn*)beta, state,
      (TOut*)o, nh, (const TIn*)ogate);
  return hipGetLastError();
}

template <typename TIn, typename TOut, bool LOGITS>
hipError_t dispatch_decode_dl(const void* q, const void* k, const void* v, const void* g,
                              const void* beta, float* state, void* o, int64_t nh, int dk, int dv,
                              const void* z, hipStream_t s) {
  if (dk == 128 && dv == 128) return launch_decode<TIn, TOut, 128, 128, LOGITS>(q, k, v, g, beta, state, o, nh, z, s);
  if (dk == 64 && dv == 64) return launch_decode<TIn, TOut, 64, 64, LOGITS>(q, k, v, g, beta, state, o, nh, z, s);
  if (dk == 64 && dv == 128) return launch_decode<TIn, TOut, 64, 128, LOGITS>(q, k, v, g, beta, state, o, nh, z, s);
  return launch_decode<TIn, TOut, 128, 64, LOGITS>(q, k, v, g, beta, state, o, nh, z, s);
}

template <typename TIn, typename TOut>
hipError_t dispatch_decode_d(const void* q, const void* k, const void* v, const void* g,
                             const void* beta, float* state, void* o, int64_t nh, int dk, int dv,
                             hipStream_t s, bool gate_logits, const void* z) {
  return gate_logits ? dispatch_decode_dl<TIn, TOut, true>(q, k, v, g, beta, state, o, nh, dk, dv, z, s)
                     : dispatch_decode_dl<TIn, TOut, false>(q, k, v, g, beta, state, o, nh, dk, dv, z, s);
}

template <typename TIn, typename TOut, bool COMMIT>
hipError_t launch_multi(const void* q, const void* k, const void* v, const void* g,
                        const void* beta, const int32_t* accept, float* state, void* o, int64_t N,
                        int64_t K, int64_t H, int dk, int dv, hipStream_t s) {
  const dim3 block(kMultiThreads);
#define KDA_MULTI(DK_, DV_)                                                                     \
  do {                                                                                          \
    auto* kern = multi_token_kernel<TIn, TOut, DK_, DV_, COMMIT>;                              \
    kern<<<dim3((unsigned)(N * H)), block, 0, s>>>(                                             \
        (const TIn*)q, (const TIn*)k, (const TIn*)v, (const TIn*)g, (const TIn*)beta, accept,   \
        state, (TOut*)o, N, K, H);                                                              \
  } while (0)
  if (dk == 128 && dv == 128) KDA_MULTI(128, 128);
  else if (dk == 64 && dv == 64) KDA_MULTI(64, 64);
  else if (dk == 64 && dv == 128) KDA_MULTI(64, 128);
  else KDA_MULTI(128, 64);
#undef KDA_MULTI
  return hipGetLastError();
}

hipError_t multi_token(const void* q, const void* k, const void* v, const void* g,
                       const void* beta, const int32_t* accept, float* state, void* o, int64_t N,
                       int64_t K, int64_t H, int dk, int dv, bool in_bf16, bool out_bf16,
                       bool commit, hipStream_t s) {
  if (commit) {
    return in_bf16 ? launch_multi<__bf16, __bf16, true>(q, k, v, g, beta, accept, state, o, N, K, H, dk, dv, s)
                   : launch_multi<float, float, true>(q, k, v, g, beta, accept, state, o, N, K, H, dk, dv, s);
  }
  if (in_bf16) {
    return out_bf16 ? launch_multi<__bf16, __bf16, false>(q, k, v, g, beta, accept, state, o, N, K, H, dk, dv, s)
                    : launch_multi<__bf16, float, false>(q, k, v, g, beta, accept, state, o, N, K, H, dk, dv, s);
  }
  return out_bf16 ? launch_multi<float, __bf16, false>(q, k, v, g, beta, accept, state, o, N, K, H, dk, dv, s)
                  : launch_multi<float, float, false>(q, k, v, g, beta, accept, state, o, N, K, H, dk, dv, s);
}

hipError_t decode_step(const void* q, const void* k, const void* v, const void* g,
                       const void* beta, float* state, void* o, int64_t nh, int dk, int dv,
                       bool in_bf16, bool out_bf16, hipStream_t s, bool gate_logits,
                       const void* z) {
  const bool L = gate_logits;
  if (in_bf16) {
    return out_bf16 ? dispatch_decode_d<__bf16, __bf16>(q, k, v, g, beta, state, o, nh, dk, dv, s, L, z)
                    : dispatch_decode_d<__bf16, float>(q, k, v, g, beta, state, o, nh, dk, dv, s, L, z);
  }
  return out_bf16 ? dispatch_decode_d<float, __bf16>(q, k, v, g, beta, state, o, nh, dk, dv, s, L, z)
                  : dispatch_decode_d<float, float>(q, k, v, g, beta, state, o, nh, dk, dv, s, L, z);
}

}  // namespace kda
