// Prefill planning and dispatch (section 3.5 of "A Taylor-Series Route to
// Linear-Time Transformers with a Fixed Number of Recurrent States", arXiv
// 2610.20637), and the exclusive scan of per-segment state sums that the
// feature-blocked prefill runs between its two passes.
//
// Which kernel a prefill call takes:
//   d = 16, n = 1, 2            single launch over 256-token segments
//                               (taylor_prefill_small.hip)
//   d = 16, n = 3, bfloat16 in,  single launch with a look-back across
//   chunk 64 or 128             segments (taylor_prefill_n3.hip)
//   everything else             feature-blocked two-pass prefill
//                               (taylor_prefill_fb.hip)
// States are additive (section 5.2): a sequence is cut into segments whose
// state sums are scanned into prefixes, so the segments run on different
// workgroups.
#include <algorithm>

#include "taylor_device.h"
#include "taylor_launch.h"

namespace taylor {

// Exclusive scan of the segment sums, in place, seeded with the caller's state:
// slot s <- state + sum_{s' < s} (segment sum s').  Slot nseg-1 never holds a
// sum (the last segment's total is not needed), only its prefix.  One float
// per thread; the loads of a block of 16 slots are issued before any store, so
// they are in flight together.
template <typename VT>
__device__ __forceinline__ void scan_slots(const VT* src, VT* slot0, size_t stride, int nseg) {
  VT run = *src;
  for (int s0 = 0; s0 < nseg; s0 += 16) {
    VT tmp[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int s = s0 + i;
      tmp[i] = (s < nseg - 1) ? slot0[(size_t)s * stride] : VT{};
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int s = s0 + i;
      if (s < nseg) slot0[(size_t)s * stride] = run;
      run += tmp[i];
    }
  }
}

__global__ __launch_bounds__(256) void segment_scan_kernel(const float* __restrict__ st_S,
                                                           const float* __restrict__ st_T,
                                                           float* __restrict__ W_S, float* __restrict__ W_T,
                                                           int D, int nseg) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int nS = D * kDV;
  if (e >= nS + D) return;
  if (e < nS)
    scan_slots(st_S + (size_t)bh * nS + e, W_S + (size_t)bh * nseg * nS + e, (size_t)nS, nseg);
  else
    scan_slots(st_T + (size_t)bh * D + (e - nS), W_T + (size_t)bh * nseg * D + (e - nS), (size_t)D, nseg);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
hipError_t launch_segment_scan(const float* st_S, const float* st_T, float* W_S, float* W_T, int D, int nseg, int BH,
                               hipStream_t stream) {
  dim3 sgrid((D * (kDV + 1) + 255) / 256, BH);
  hipLaunchKernelGGL(segment_scan_kernel, sgrid, dim3(256), 0, stream, st_S, st_T, W_S, W_T, D, nseg);
  return hipGetLastError();
}

PrefillPlan plan_prefill(int BH, int N, int d, int n, int chunk) {
  PrefillPlan p;
  if (BH <= 0 || N <= 0 || chunk <= 0) return p;
  if (d == 16 && n <= 2) {  // fixed segments of 128 or 256 tokens, 16-token chunks inside
    const int L = small_segment_tokens(n);
    p.nchunks = (N + 15) / 16;
    p.chunks_per_seg = L / 16;
    p.nseg = (N + L - 1) / L;
    p.workspace_floats = prefill_small_workspace_floats(BH, N, n);
    return p;
  }
  p.nchunks = (N + chunk - 1) / chunk;
  // Every segment is split into feature blocks, one workgroup each; aim at one
  // round of workgroups (two per CU on a 256-CU part, one per CU for 128-token
  // chunks, which fill an LDS on their own) and never more (a second, partial
  // round would cost as much as the first).
  const int blocks = prefill_fb_blocks(d, n);
  const int target = chunk >= 128 ? 256 : 512;
  int nseg = target / (BH * blocks);
  if (nseg < 1) nseg = 1;
  if (nseg > p.nchunks) nseg = p.nchunks;
  p.chunks_per_seg = (p.nchunks + nseg - 1) / nseg;
  p.nseg = (p.nchunks + p.chunks_per_seg - 1) / p.chunks_per_seg;
  const int D = state_width_d(d, n);
  p.workspace_floats = p.nseg > 1 ? (size_t)BH * p.nseg * D * (kDV + 1) : 0;
  // d = 16, n = 3 with bfloat16 inputs takes the look-back kernel, whose
  // workspace is larger; the size does not depend on the input type, so
  // cover both
  if (d == 16 && n == 3) p.workspace_floats = std::max(p.workspace_floats, prefill_n3_workspace_floats(BH, p.nseg));
  const size_t out = prefill_fb_output_floats(BH, N, d, n);
  if (out > 0) p.workspace_floats = (p.workspace_floats + 3) / 4 * 4 + out;  // 16-byte aligned partial outputs
  return p;
}

bool prefill_supported(int d, int n, int chunk, bool in_bf16) {
  if (d == 32 || d == 64) return n >= 1 && n <= 3 && (chunk == 32 || chunk == 64);
  if (d != 16) return false;
  if (n >= 4 && n <= 6) return chunk == 32 || chunk == 64;
  if (n < 1 || n > 3) return false;
  if (in_bf16) return chunk == 32 || chunk == 64 || chunk == 128;
  return chunk == 32 || chunk == 64;
}

hipError_t launch_prefill(const PrefillArgs& a) {
  if (a.d == kD && a.n <= 2) return launch_prefill_small(a);
  if (a.d == kD && a.n == 3 && a.in_bf16 && (a.chunk == 64 || a.chunk == 128)) return launch_prefill_n3_bf16(a);
  return launch_prefill_fb(a);
}

}  // namespace taylor
