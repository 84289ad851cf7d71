// Eviction-fed hybrid decode: a FIFO window of the last W key-value pairs read
// by exact softmax attention, and a memory written only with the pairs the
// window evicts ("Tensor Cache: Eviction-conditioned Associative Memory for
// Transformers", sections 3.1-3.2), where the memory is the n-term Taylor
// state of "A Taylor-Series Route to Linear-Time Transformers with a Fixed
// Number of Recurrent States" (Eq. (6)-(7), read through Eq. (5)).  Every
// earlier token feeds exactly one path, and both share one normaliser:
//   o_t = (sum_{window} e^{q.k_i/a} [v_i;1] + phi_hat(q) A)[:d_v] / (same)[d_v],
// A holding the evicted tokens.
//
// One workgroup of 256 threads per (b, h), d = 16, d_v = 64, n <= 3, W <= 1024:
//   * the token leaving the window (the one in ring slot pos % W, once
//     pos >= W) is added to the state, A += phi(k_old) [v_old; 1]^T, in the
//     same pass over the state that reads phi_hat(q) A (the state is streamed
//     once: 16 threads per 256-byte row);
//   * the window (the new token and the W - 1 before it) is read with a
//     running maximum m per thread (4 threads per key: 4 of its 16 dimensions,
//     16 of the 64 value columns), merged across lanes and waves by the
//     rescaling rule; m starts at 0, so the shared factor e^{-m} <= 1 also
//     scales the state's part;
//   * the new token goes into ring slot pos % W last (that slot's old token
//     was read into LDS first).
#include "taylor_device.h"
#include "taylor_launch.h"

namespace taylor {
namespace hy {

__constant__ FeatureTable kTab = make_feature_table();
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kMaxWindow = 1024;

template <typename T> struct V4;
template <> struct V4<float> {
  static __device__ __forceinline__ void load(const float* p, float (&x)[4]) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
  }
};
template <> struct V4<uint16_t> {
  static __device__ __forceinline__ void load(const uint16_t* p, float (&x)[4]) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    x[0] = __uint_as_float(u.x << 16); x[1] = __uint_as_float(u.x & 0xFFFF0000u);
    x[2] = __uint_as_float(u.y << 16); x[3] = __uint_as_float(u.y & 0xFFFF0000u);
  }
};

// (m, l, o) <- merge with (m2, l2, o2): weights relative to 2^m; m >= 0 on both sides.
template <int NV>
__device__ __forceinline__ void merge(float& m, float& l, float (&o)[NV], float m2, float l2, const float (&o2)[NV]) {
  const float M = fmaxf(m, m2);
  const float c1 = exp2f(m - M), c2 = exp2f(m2 - M);
  l = l * c1 + l2 * c2;
#pragma unroll
  for (int i = 0; i < NV; ++i) o[i] = o[i] * c1 + o2[i] * c2;
  m = M;
}

template <int NT, typename TIN, typename TOUT>
__global__ __launch_bounds__(256) void hybrid_decode_kernel(const TIN* __restrict__ q, const TIN* __restrict__ k,
                                                            const TIN* __restrict__ v, TOUT* __restrict__ o,
                                                            float* __restrict__ S, float* __restrict__ T,
                                                            TIN* __restrict__ wk, TIN* __restrict__ wv, int pos,
                                                            int W, float inv_a) {
  constexpr int D = state_width(NT);
  constexpr int kRows = (D + 15) / 16;
  const int bh = blockIdx.x, tid = threadIdx.x, c4 = tid & 15, rg = tid >> 4;
  const int lane = tid & 63, wave = tid >> 6;
  float* __restrict__ Sh = S + (size_t)bh * D * kDV;
  float* __restrict__ Th = T + (size_t)bh * D;
  const size_t ring = (size_t)bh * W;
  const int slot = pos % W;
  const bool evict = pos >= W;  // uniform

  // the new token (threads 0..95) and the evicted one (96..175) into LDS
  __shared__ float xq[kD], xk[kD], xko[kD];
  __shared__ __align__(16) float xv[kDV], xvo[kDV];
  __shared__ float phq[D], phk[D];
  {
    float x = 0.f;
    if (tid < kD) x = Elem<TIN>::load(q, (size_t)bh * kD + tid);
    else if (tid < 2 * kD) x = Elem<TIN>::load(k, (size_t)bh * kD + tid - kD);
    else if (tid < 2 * kD + kDV) x = Elem<TIN>::load(v, (size_t)bh * kDV + tid - 2 * kD);
    else if (tid < 3 * kD + kDV) x = Elem<TIN>::load(wk, (ring + slot) * kD + tid - 2 * kD - kDV);
    else if (tid < 3 * kD + 2 * kDV) x = Elem<TIN>::load(wv, (ring + slot) * kDV + tid - 3 * kD - kDV);
    if (tid < kD) xq[tid] = x;
    else if (tid < 2 * kD) xk[tid - kD] = x;
    else if (tid < 2 * kD + kDV) xv[tid - 2 * kD] = x;
    else if (tid < 3 * kD + kDV) xko[tid - 2 * kD - kDV] = x;
    else if (tid < 3 * kD + 2 * kDV) xvo[tid - 3 * kD - kDV] = x;
  }
  // this thread's state rows (clamped past D; unused there)
  float4 sv[kRows];
#pragma unroll
  for (int i = 0; i < kRows; ++i)
    sv[i] = *reinterpret_cast<const float4*>(Sh + (size_t)min(rg + 16 * i, D - 1) * kDV + 4 * c4);
  const float tv = Th[min(tid, D - 1)];
  __syncthreads();
  const float a2 = inv_a * inv_a;
  if (tid < D) {
    phq[tid] = feature_value(kTab, tid, xq, make_float4(1.0f, inv_a, 0.5f * a2, 0.0f));
    phk[tid] = feature_value(kTab, tid, xko, make_float4(1.0f, 1.0f, 1.0f, 1.0f));
  }
  __syncthreads();

  // ---- the state: add the evicted token, then read
  const float4 vo = *reinterpret_cast<const float4*>(&xvo[4 * c4]);
  float4 sacc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int r = rg + 16 * i;
    if (r < D) {
      float4 s = sv[i];
      if (evict) {
        const float pk = phk[r];
        s.x += pk * vo.x; s.y += pk * vo.y; s.z += pk * vo.z; s.w += pk * vo.w;
        *reinterpret_cast<float4*>(Sh + (size_t)r * kDV + 4 * c4) = s;
      }
      const float pq = phq[r];
      sacc.x += pq * s.x; sacc.y += pq * s.y; sacc.z += pq * s.z; sacc.w += pq * s.w;
    }
  }
  float sden = 0.f;
  if (tid < D) {
    float t = tv;
    if (evict) {
      t += phk[tid];
      Th[tid] = t;
    }
    sden = phq[tid] * t;
  }

  // ---- the window: keys at positions max(0, pos - W + 1) .. pos
  const int quad = tid & 3, kslot = tid >> 2;  // 64 key slots, 4 threads per key
  const int nw = min(pos + 1, W);
  float qv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) qv[i] = xq[4 * quad + i] * (inv_a * kLog2e);  // scores in log2 units
  float m = 0.f, l = 0.f, acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  for (int j0 = 0; j0 < nw; j0 += 64) {  // uniform trip count
    const int j = j0 + kslot;           // j-th window key: position pos - j
    const bool valid = j < nw;
    const int sl = ((pos - min(j, nw - 1)) % W + W) % W;
    float kk[4], vv[16];
    if (j == 0) {  // the new token, from LDS (its slot still holds the evicted one)
#pragma unroll
      for (int i = 0; i < 4; ++i) kk[i] = xk[4 * quad + i];
#pragma unroll
      for (int i = 0; i < 16; ++i) vv[i] = xv[16 * quad + i];
    } else {
      V4<TIN>::load(wk + (ring + sl) * kD + 4 * quad, kk);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x4[4];
        V4<TIN>::load(wv + (ring + sl) * kDV + 16 * quad + 4 * e, x4);
#pragma unroll
        for (int i = 0; i < 4; ++i) vv[4 * e + i] = x4[i];
      }
    }
    float s = qv[0] * kk[0] + qv[1] * kk[1] + qv[2] * kk[2] + qv[3] * kk[3];
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if (valid) {
      const float mn = fmaxf(m, s);
      const float c = exp2f(m - mn), p = exp2f(s - mn);
      l = l * c + p;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = acc[i] * c + p * vv[i];
      m = mn;
    }
  }
  // merge the 16 key slots of a wave (lanes 4, 8, 16, 32 apart share columns)
#pragma unroll
  for (int off = 4; off <= 32; off <<= 1) {
    float o2[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) o2[i] = __shfl_xor(acc[i], off);
    const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
    merge<16>(m, l, acc, m2, l2, o2);
  }
  // the state's partial reads: rows of 16 threads (lanes 16 and 32 apart share columns)
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
    sacc.x += __shfl_xor(sacc.x, off);
    sacc.y += __shfl_xor(sacc.y, off);
    sacc.z += __shfl_xor(sacc.z, off);
    sacc.w += __shfl_xor(sacc.w, off);
  }
#pragma unroll
  for (int off = 1; off <= 32; off <<= 1) sden += __shfl_xor(sden, off);
  __shared__ float wred[4][4][18];         // [wave][quad][m, l, 16 values]
  __shared__ __align__(16) float sred[4][kDV];
  __shared__ float sdred[4];
  if (lane < 4) {
    wred[wave][lane][0] = m;
    wred[wave][lane][1] = l;
#pragma unroll
    for (int i = 0; i < 16; ++i) wred[wave][lane][2 + i] = acc[i];
  }
  if (lane < 16) *reinterpret_cast<float4*>(&sred[wave][4 * lane]) = sacc;
  if (lane == 0) sdred[wave] = sden;
  __syncthreads();
  if (tid < kDV) {
    const int qd = tid >> 4, i = tid & 15;
    float mm = wred[0][qd][0], ll = wred[0][qd][1], oo[1] = {wred[0][qd][2 + i]};
#pragma unroll
    for (int wv2 = 1; wv2 < 4; ++wv2) {
      const float o2[1] = {wred[wv2][qd][2 + i]};
      merge<1>(mm, ll, oo, wred[wv2][qd][0], wred[wv2][qd][1], o2);
    }
    // the state's part carries the same factor 2^{-m} as the window's weights
    const float f = exp2f(-mm);
    const float y = oo[0] + f * (sred[0][tid] + sred[1][tid] + sred[2][tid] + sred[3][tid]);
    const float den = ll + f * (sdred[0] + sdred[1] + sdred[2] + sdred[3]);
    Elem<TOUT>::store(o, (size_t)bh * kDV + tid, y / den);
  }
  // the new token into its ring slot (the slot's old token was read above)
  if (tid >= kD && tid < 2 * kD) Elem<TIN>::store(wk, (ring + slot) * kD + tid - kD, xk[tid - kD]);
  else if (tid >= 2 * kD && tid < 2 * kD + kDV)
    Elem<TIN>::store(wv, (ring + slot) * kDV + tid - 2 * kD, xv[tid - 2 * kD]);
}

// Ring slots from a context: token i of the last min(N, W) of k, v [BH, N, .]
// goes to slot i % W.
template <typename TIN>
__global__ __launch_bounds__(256) void fill_window_kernel(const TIN* __restrict__ k, const TIN* __restrict__ v,
                                                          TIN* __restrict__ wk, TIN* __restrict__ wv, int N, int W) {
  const int bh = blockIdx.y;
  const int nw = min(N, W);
  const size_t per = (size_t)nw * (kD + kDV);
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < per; e += (size_t)gridDim.x * 256) {
    const int j = (int)(e / (kD + kDV)), c = (int)(e % (kD + kDV));
    const int i = N - nw + j;  // position
    const int sl = i % W;
    if (c < kD) wk[((size_t)bh * W + sl) * kD + c] = k[((size_t)bh * N + i) * kD + c];
    else wv[((size_t)bh * W + sl) * kDV + c - kD] = v[((size_t)bh * N + i) * kDV + c - kD];
  }
}

template <int NT, typename TIN, typename TOUT>
hipError_t launch_t(const HybridDecodeArgs& a) {
  constexpr int D = state_width(NT);
  hipLaunchKernelGGL((hybrid_decode_kernel<NT, TIN, TOUT>), dim3(a.BH), dim3(256), 0, a.stream,
                     static_cast<const TIN*>(a.q), static_cast<const TIN*>(a.k), static_cast<const TIN*>(a.v),
                     static_cast<TOUT*>(a.o), a.state, a.state + (size_t)a.BH * D * kDV,
                     static_cast<TIN*>(a.win_k), static_cast<TIN*>(a.win_v), a.pos, a.window, 1.0f / a.a);
  return hipGetLastError();
}

template <int NT>
hipError_t launch_n(const HybridDecodeArgs& a) {
  if (a.in_bf16) return a.out_bf16 ? launch_t<NT, uint16_t, uint16_t>(a) : launch_t<NT, uint16_t, float>(a);
  return a.out_bf16 ? launch_t<NT, float, uint16_t>(a) : launch_t<NT, float, float>(a);
}

}  // namespace hy

int hybrid_max_window() { return hy::kMaxWindow; }

hipError_t launch_hybrid_decode(const HybridDecodeArgs& a) {
  switch (a.n) {
    case 1: return hy::launch_n<1>(a);
    case 2: return hy::launch_n<2>(a);
    case 3: return hy::launch_n<3>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_hybrid_fill_window(const void* k, const void* v, void* wk, void* wv, int BH, int N, int W,
                                     bool in_bf16, hipStream_t stream) {
  const size_t per = (size_t)(N < W ? N : W) * (kD + kDV);
  const unsigned gx = (unsigned)((per + 255) / 256 < 64 ? (per + 255) / 256 : 64);
  if (in_bf16)
    hipLaunchKernelGGL(hy::fill_window_kernel<uint16_t>, dim3(gx, BH), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), static_cast<uint16_t*>(wk),
                       static_cast<uint16_t*>(wv), N, W);
  else
    hipLaunchKernelGGL(hy::fill_window_kernel<float>, dim3(gx, BH), dim3(256), 0, stream,
                       static_cast<const float*>(k), static_cast<const float*>(v), static_cast<float*>(wk),
                       static_cast<float*>(wv), N, W);
  return hipGetLastError();
}

}  // namespace taylor
