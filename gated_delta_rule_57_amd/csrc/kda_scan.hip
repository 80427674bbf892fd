// Entry states of sequence segments from their summaries.
//
// The state map of one segment is affine in its entry state: S_out = P S_in + Z,
// with Z the state the segment reaches from a zero state and P (d_k x d_k) the
// product of its per-token transitions, (I - beta k k^T) Diag(exp g').  Cutting
// a long sequence into segments, summarising every segment independently and
// chaining the summaries with a prefix scan recovers every segment's entry
// state; this is the decomposition the orkas.ai blog "Kimi K3 architecture"
// describes for spreading one sequence over devices (section "The cost is paid
// in the serving stack").  Here the segments share one GPU: the summaries come
// from the chunk kernel's summary pass and this kernel runs the scan.
//
// One workgroup per (b, h, 32 state columns); the scan is serial over segments.
// P_j is staged through shared memory in blocks of 64 of its columns; each
// thread owns RB rows x 4 columns of the running state.  float32 FMA throughout.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int DK, int DV>
__global__ void __launch_bounds__(256) segment_scan_kernel(const float* seg_z,
                                                           const float* seg_p, float* seg_in,
                                                           int64_t H, int64_t nseg) {
  constexpr int NC = 32;                   // state columns per workgroup
  constexpr int KB = 64;                   // P columns per shared-memory block
  constexpr int RB = DK * NC / (256 * 4);  // state rows per thread
  static_assert(RB * 4 * 256 == DK * NC && DK % KB == 0, "layout");
  __shared__ float sP[DK][KB + 1];  // one column block of P_j (row-major, padded)
  __shared__ __align__(16) float sS[DK][NC + 4];

  const int64_t unit = blockIdx.x / (DV / NC);
  const int cb = (int)(blockIdx.x % (DV / NC)) * NC;
  const int64_t b = unit / H, h = unit % H;
  const int tid = threadIdx.x, cq = 4 * (tid % 8), r0 = RB * (tid / 8);
  auto blk = [&](auto* base, int64_t j) {
    return base + ((b * nseg + j) * H + h) * (int64_t)DK * DV + cb;
  };

  // slot 1: the state after segment 0 (its summary walked it from the initial
  // state); slot 0 stays unused, segment 0 being walked by the summary pass itself
  for (int e = tid; e < DK * NC / 4; e += 256) {
    const int r = e / (NC / 4), c = 4 * (e % (NC / 4));
    const float4 z = *reinterpret_cast<const float4*>(blk(seg_z, 0) + (int64_t)r * DV + c);
    *reinterpret_cast<float4*>(blk(seg_in, 1) + (int64_t)r * DV + c) = z;
    *reinterpret_cast<float4*>(&sS[r][c]) = z;
  }

  for (int64_t j = 1; j + 1 < nseg; ++j) {
    const float* Pj = seg_p + ((b * nseg + j) * H + h) * (int64_t)DK * DK;
    const float* Zj = blk(seg_z, j);
    float4 acc[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i)
      acc[i] = *reinterpret_cast<const float4*>(Zj + (int64_t)(r0 + i) * DV + cq);
    for (int k0 = 0; k0 < DK; k0 += KB) {
      __syncthreads();  // sS complete; the previous block of P consumed
      for (int e = tid; e < DK * KB; e += 256) {
        const int r = e / KB, k = e % KB;
        sP[r][k] = Pj[(int64_t)r * DK + k0 + k];
      }
      __syncthreads();
#pragma unroll 8
      for (int k = 0; k < KB; ++k) {
        const float4 s = *reinterpret_cast<const float4*>(&sS[k0 + k][cq]);
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          const float pv = sP[r0 + i][k];
          acc[i].x = fmaf(pv, s.x, acc[i].x);
          acc[i].y = fmaf(pv, s.y, acc[i].y);
          acc[i].z = fmaf(pv, s.z, acc[i].z);
          acc[i].w = fmaf(pv, s.w, acc[i].w);
        }
      }
    }
    __syncthreads();  // every thread is done reading sS
    float* out = blk(seg_in, j + 1);
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      *reinterpret_cast<float4*>(&sS[r0 + i][cq]) = acc[i];
      *reinterpret_cast<float4*>(out + (int64_t)(r0 + i) * DV + cq) = acc[i];
    }
  }
}

template <int DK, int DV>
static hipError_t launch_scan(const float* seg_z, const float* seg_p,
                              float* seg_in, int64_t B, int64_t H, int64_t nseg, hipStream_t s) {
  const int64_t grid = B * H * (DV / 32);
  segment_scan_kernel<DK, DV><<<dim3((unsigned)grid), dim3(256), 0, s>>>(seg_z, seg_p, seg_in,
                                                                         H, nseg);
  return hipGetLastError();
}

hipError_t segment_scan(const float* seg_z, const float* seg_p, float* seg_in,
                        int64_t B, int64_t H, int64_t nseg, int dk, int dv, hipStream_t s) {
  if (dk == 128 && dv == 128) return launch_scan<128, 128>(seg_z, seg_p, seg_in, B, H, nseg, s);
  if (dk == 128 && dv == 64) return launch_scan<128, 64>(seg_z, seg_p, seg_in, B, H, nseg, s);
  if (dk == 64 && dv == 128) return launch_scan<64, 128>(seg_z, seg_p, seg_in, B, H, nseg, s);
  return launch_scan<64, 64>(seg_z, seg_p, seg_in, B, H, nseg, s);
}

}  // namespace kda
