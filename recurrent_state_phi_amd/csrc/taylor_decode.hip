// Single-token decode step (section 3.3, Eq. (7), then the readout of Eq. (5), of
// "A Taylor-Series Route to Linear-Time Transformers with a Fixed Number of
// Recurrent States", arXiv 2610.20637).
//
// Per head: A <- A + phi(k) [v; 1]^T, then y = phi_hat(q)^T A and o = y[:dv] / y[dv],
// with phi_hat(q) = alpha_m phi_m(q), alpha_m = 1 / (m! a^m).  The state is
// streamed from HBM exactly once (read, add the rank-one term, write back,
// accumulate the read), so the kernel is bound by HBM bandwidth: 2 * 4 * D * 65
// bytes per head per step against about 4 * D * 65 flops.
//
// One 256-thread workgroup per (b, h).  Thread layout for the S block
// [D][64]: 16 threads cover one 256-byte row with float4 accesses, 16 rows are
// in flight per pass, so every wave reads four full rows per instruction.
// For n <= 3 (at most 153 rows, 10 per thread) every thread issues all of its
// state loads first, so they are in flight while q, k and v are fetched and
// the features are formed; the larger n = 4 state is streamed in a loop.
#include "taylor_device.h"
#include "taylor_launch.h"

namespace taylor {

__constant__ FeatureTable kFeatTab = make_feature_table();

static __device__ RowTable<16, 5> kRows16 = make_row_table<16, 5>();  // d = 16, n = 5, 6
static __device__ RowTable<32, 2> kRows32 = make_row_table<32, 2>();  // d = 32, n <= 3
static __device__ RowTable<64, 2> kRows64 = make_row_table<64, 2>();  // d = 64, n <= 3

template <int KD>
__device__ __forceinline__ uint32_t row_code(int f) {
  if constexpr (KD == 16) return kRows16.code[f];
  else if constexpr (KD == 32) return kRows32.code[f];
  else return kRows64.code[f];
}
template <int KD> constexpr int table_orders() { return KD == 16 ? 5 : 2; }

// Sum of the partial reads of the NWV * 64 threads (row groups of 16 threads:
// 4 inside a wave, lanes 16 apart, then the NWV waves) and o = y[:d_v] / y[d_v].
// acc holds this thread's 4 columns of y, dacc its part of the normaliser.
template <typename TOUT, int NWV = 4>
__device__ __forceinline__ void finish_read(float4 acc, float dacc, TOUT* __restrict__ o, int bh, int tid) {
  __shared__ __align__(16) float red[NWV][kDV];
  __shared__ float red_den[NWV];
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
    acc.x += __shfl_xor(acc.x, off);
    acc.y += __shfl_xor(acc.y, off);
    acc.z += __shfl_xor(acc.z, off);
    acc.w += __shfl_xor(acc.w, off);
  }
#pragma unroll
  for (int off = 1; off <= 32; off <<= 1) dacc += __shfl_xor(dacc, off);
  if (lane < 16) *reinterpret_cast<float4*>(&red[wave][4 * lane]) = acc;
  if (lane == 0) red_den[wave] = dacc;
  __syncthreads();
  if (tid < kDV) {
    float y = red[0][tid], den = red_den[0];
#pragma unroll
    for (int i = 1; i < NWV; ++i) {
      y += red[i][tid];
      den += red_den[i];
    }
    Elem<TOUT>::store(o, (size_t)bh * kDV + tid, y / den);
  }
}

template <int NT, typename TIN, typename TOUT>
__global__ __launch_bounds__(256) void decode_step_kernel(const TIN* __restrict__ q, const TIN* __restrict__ k,
                                                          const TIN* __restrict__ v, TOUT* __restrict__ o,
                                                          float* __restrict__ S, float* __restrict__ T,
                                                          float inv_a) {
  constexpr int D = state_width(NT);
  constexpr int kRows = (D + 15) / 16;      // rows per thread in the S block
  constexpr bool kPrefetch = kRows <= 12;   // whole share held in registers
  static_assert(!kPrefetch || D <= 256, "one feature row and one T entry per thread");
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  float* __restrict__ Sh = S + (size_t)bh * D * kDV;
  float* __restrict__ Th = T + (size_t)bh * D;
  const int c4 = tid & 15, rg = tid >> 4;

  // Loads in issue order: this thread's element of q, k or v and its feature
  // row (waited for first), then its share of the state (waited for last).
  float xin = 0.f;
  if (tid < kD) xin = Elem<TIN>::load(q, (size_t)bh * kD + tid);
  else if (tid < 2 * kD) xin = Elem<TIN>::load(k, (size_t)bh * kD + tid - kD);
  else if (tid < 2 * kD + kDV) xin = Elem<TIN>::load(v, (size_t)bh * kDV + tid - 2 * kD);
  uint32_t fcode = 0;
  float fweight = 0.f;
  // Every load below is issued unconditionally (row indices past the state are
  // clamped to its last row, and those values are not used), so the waits
  // that follow count exactly the loads ahead of them.
  const int frow = tid < D ? tid : D - 1;
  if constexpr (kPrefetch) {
    fcode = kFeatTab.code[frow];
    fweight = kFeatTab.weight[frow];
  }
  float4 sv[kPrefetch ? kRows : 1];
  float tv = 0.f;
  if constexpr (kPrefetch) {
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      const int r = rg + 16 * i < D ? rg + 16 * i : D - 1;
      sv[i] = *reinterpret_cast<const float4*>(Sh + (size_t)r * kDV + 4 * c4);
    }
    tv = Th[frow];
  }

  __shared__ float xq[kD], xk[kD];
  __shared__ __align__(16) float vs[kDV];
  __shared__ float phq[D], phk[D];

  if (tid < kD) xq[tid] = xin;
  else if (tid < 2 * kD) xk[tid - kD] = xin;
  else if (tid < 2 * kD + kDV) vs[tid - 2 * kD] = xin;
  __syncthreads();

  const float a2 = inv_a * inv_a;
  const float4 alpha_q = make_float4(1.0f, inv_a, 0.5f * a2, a2 * inv_a * (1.0f / 6.0f));
  const float4 alpha_k = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
  if constexpr (kPrefetch) {
    if (tid < D) {
      phq[tid] = feature_value(fcode, fweight, xq, alpha_q);
      phk[tid] = feature_value(fcode, fweight, xk, alpha_k);
    }
  } else {
    for (int f = tid; f < D; f += 256) {
      phq[f] = feature_value(kFeatTab, f, xq, alpha_q);
      phk[f] = feature_value(kFeatTab, f, xk, alpha_k);
    }
  }
  __syncthreads();

  // S block: rank-one update then read, one pass over [D][64].
  const float4 vv = *reinterpret_cast<const float4*>(&vs[4 * c4]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto update_read = [&](int r, float4 s) {
    const float pk = phk[r];
    s.x += pk * vv.x; s.y += pk * vv.y; s.z += pk * vv.z; s.w += pk * vv.w;
    *reinterpret_cast<float4*>(Sh + (size_t)r * kDV + 4 * c4) = s;
    const float pq = phq[r];
    acc.x += pq * s.x; acc.y += pq * s.y; acc.z += pq * s.z; acc.w += pq * s.w;
  };
  float dacc = 0.f;
  if constexpr (kPrefetch) {
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      const int r = rg + 16 * i;
      if (r < D) update_read(r, sv[i]);
    }
    // T block (the ones-column): same update and read.
    if (tid < D) {
      const float t = tv + phk[tid];
      Th[tid] = t;
      dacc = phq[tid] * t;
    }
  } else {
#pragma unroll 4
    for (int r = rg; r < D; r += 16) update_read(r, *reinterpret_cast<const float4*>(Sh + (size_t)r * kDV + 4 * c4));
    for (int r = tid; r < D; r += 256) {
      const float t = Th[r] + phk[r];
      Th[r] = t;
      dacc += phq[r] * t;
    }
  }

  finish_read<TOUT>(acc, dacc, o, bh, tid);
}

// Orders up to 5 (n = 5, 6: 4,845 or 20,349 rows; the two feature vectors of
// n = 6 alone would take 163 KB of LDS): 512 threads per head (32 row groups,
// so 16 waves per CU keep the long stream of state rows in flight), the same
// one pass over the state,
// with the features phi(k)_r and phi_hat(q)_r formed from the row table into
// LDS one piece of kPiece rows at a time, one row per thread.  The state rows
// are streamed in double-buffered batches of 8 per thread; the loads of the
// next batch are issued before a piece's features are formed, so they stay in
// flight across it.  The ones-column T of a piece is updated and read by the
// thread that forms the piece's row.
constexpr int kWideThreads = 512;

template <int NT, int KD, typename TIN, typename TOUT>
__global__ __launch_bounds__(kWideThreads) void decode_step_wide_kernel(const TIN* __restrict__ q, const TIN* __restrict__ k,
                                                               const TIN* __restrict__ v, TOUT* __restrict__ o,
                                                               float* __restrict__ S, float* __restrict__ T,
                                                               float inv_a) {
  constexpr int D = state_width_d(KD, NT);
  constexpr int MAXM = table_orders<KD>();
  static_assert(2 * KD + kDV <= kWideThreads, "one thread per element of q, k and v");
  constexpr int kB = 8;                              // rows per thread per batch
  constexpr int kGroups = kWideThreads / 16;        // row groups of 16 threads
  constexpr int kBatchRows = kGroups * kB;           // rows per batch (all threads)
  constexpr int kPiece = 2048;                       // rows per feature piece
  static_assert(kPiece % kBatchRows == 0, "pieces hold whole batches");
  constexpr int kBatches = (D + kBatchRows - 1) / kBatchRows;
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  float* __restrict__ Sh = S + (size_t)bh * D * kDV;
  float* __restrict__ Th = T + (size_t)bh * D;
  const int c4 = tid & 15, rg = tid >> 4;

  __shared__ float xq[KD], xk[KD];
  __shared__ __align__(16) float vs[kDV];
  __shared__ float phq[kPiece], phk[kPiece];
  if (tid < KD) xq[tid] = Elem<TIN>::load(q, (size_t)bh * KD + tid);
  else if (tid < 2 * KD) xk[tid - KD] = Elem<TIN>::load(k, (size_t)bh * KD + tid - KD);
  else if (tid < 2 * KD + kDV) vs[tid - 2 * KD] = Elem<TIN>::load(v, (size_t)bh * kDV + tid - 2 * KD);

  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float dacc = 0.f;
  // Every load is issued (row indices past the state clamped to its last row,
  // values unused).
  float4 cur[kB], nxt[kB];
  auto load_batch = [&](int b, float4 (&sv)[kB]) {
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      const int r0 = b * kBatchRows + rg + kGroups * i;
      const int r = r0 < D ? r0 : D - 1;
      sv[i] = *reinterpret_cast<const float4*>(Sh + (size_t)r * kDV + 4 * c4);
    }
  };
  load_batch(0, cur);
  __syncthreads();  // q, k, v in LDS
  const float4 vv = *reinterpret_cast<const float4*>(&vs[4 * c4]);
  int p0 = 0;  // first row of the piece whose features are in LDS
  for (int b = 0; b < kBatches; ++b) {
    if (b + 1 < kBatches) load_batch(b + 1, nxt);
    if ((b * kBatchRows) % kPiece == 0) {  // uniform: a new piece starts
      p0 = b * kBatchRows;
      __syncthreads();  // the previous piece's features are no longer read
      for (int f = tid; f < kPiece && p0 + f < D; f += kWideThreads) {
        const int r = p0 + f;
        const float tr = Th[r];
        const uint32_t c = row_code<KD>(r);
        const float pk = row_feature_value<KD, MAXM>(c, xk, 1.0f);
        const float pq = row_feature_value<KD, MAXM>(c, xq, alpha_of(inv_a, c));
        phk[f] = pk;
        phq[f] = pq;
        const float t = tr + pk;  // T block (the ones-column): update, then read
        Th[r] = t;
        dacc += pq * t;
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      const int r = b * kBatchRows + rg + kGroups * i;
      if (r < D) {
        float4 s = cur[i];
        const float pk = phk[r - p0], pq = phq[r - p0];
        s.x += pk * vv.x; s.y += pk * vv.y; s.z += pk * vv.z; s.w += pk * vv.w;
        *reinterpret_cast<float4*>(Sh + (size_t)r * kDV + 4 * c4) = s;
        acc.x += pq * s.x; acc.y += pq * s.y; acc.z += pq * s.z; acc.w += pq * s.w;
      }
    }
#pragma unroll
    for (int i = 0; i < kB; ++i) cur[i] = nxt[i];
  }
  finish_read<TOUT, kWideThreads / 64>(acc, dacc, o, bh, tid);
}

// d = 16, n <= 4: decode_step_kernel; d = 16, n = 5, 6 and d = 32, 64:
// decode_step_wide_kernel.
template <int NT, int KD, typename TIN, typename TOUT>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  const int D = state_width_d(KD, NT);
  float* S = a.state;
  float* T = a.state + (size_t)a.BH * D * kDV;
  if constexpr (KD == kD && NT <= 4)
    hipLaunchKernelGGL((decode_step_kernel<NT, TIN, TOUT>), dim3(a.BH), dim3(256), 0, a.stream,
                       static_cast<const TIN*>(a.q), static_cast<const TIN*>(a.k), static_cast<const TIN*>(a.v),
                       static_cast<TOUT*>(a.o), S, T, 1.0f / a.a);
  else
    hipLaunchKernelGGL((decode_step_wide_kernel<NT, KD, TIN, TOUT>), dim3(a.BH), dim3(kWideThreads), 0, a.stream,
                       static_cast<const TIN*>(a.q), static_cast<const TIN*>(a.k), static_cast<const TIN*>(a.v),
                       static_cast<TOUT*>(a.o), S, T, 1.0f / a.a);
  return hipGetLastError();
}

template <int NT, int KD>
static hipError_t launch_decode_n(const DecodeArgs& a) {
  if (!a.in_bf16 && !a.out_bf16) return launch_decode_t<NT, KD, float, float>(a);
  if (!a.in_bf16 && a.out_bf16) return launch_decode_t<NT, KD, float, uint16_t>(a);
  if (a.in_bf16 && !a.out_bf16) return launch_decode_t<NT, KD, uint16_t, float>(a);
  return launch_decode_t<NT, KD, uint16_t, uint16_t>(a);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, size_t n) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) p[i] = 0.0f;
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a) {
  if (a.d == 32 || a.d == 64) {
    switch (a.n) {
      case 1: return a.d == 32 ? launch_decode_n<1, 32>(a) : launch_decode_n<1, 64>(a);
      case 2: return a.d == 32 ? launch_decode_n<2, 32>(a) : launch_decode_n<2, 64>(a);
      case 3: return a.d == 32 ? launch_decode_n<3, 32>(a) : launch_decode_n<3, 64>(a);
    }
    return hipErrorInvalidValue;
  }
  switch (a.n) {
    case 1: return launch_decode_n<1, kD>(a);
    case 2: return launch_decode_n<2, kD>(a);
    case 3: return launch_decode_n<3, kD>(a);
    case 4: return launch_decode_n<4, kD>(a);
    case 5: return launch_decode_n<5, kD>(a);
    case 6: return launch_decode_n<6, kD>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace taylor
