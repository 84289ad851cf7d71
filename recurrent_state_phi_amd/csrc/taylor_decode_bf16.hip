// Decode against a state stored in bfloat16 (section 5.8 of "A Taylor-Series
// Route to Linear-Time Transformers with a Fixed Number of Recurrent States",
// arXiv 2610.20637, sizes the states in bfloat16), for n <= 3 at d = 16.
//
// A state kept in bfloat16 and updated token by token loses most of every
// increment: a row of S holds a sum of tens of thousands of terms, and one
// token's term is below half a bfloat16 unit of it, so it rounds away (after
// a 65,536-token context, 256 such steps put the outputs 4-6% off).  Here the
// state is split instead:
//   * a bfloat16 base of S (the D x d_v part, 2 bytes per element) and a
//     float32 T (the ones-column, D floats: it holds the token count, which
//     bfloat16 cannot advance past 256);
//   * an exact window of the last `step + 1 <= K` tokens (their k and v as
//     given), read with the same polynomial weights p_n(q.k / a) as the state
//     (Eq. (1)-(2) for those keys, computed directly);
//   * every K tokens the window is folded into the base, S <- round(S +
//     sum_window phi(k) v^T) and T <- T + sum_window phi(k) (Eq. (6)-(7) summed
//     over the window): one rounding per K tokens instead of one per token.
// The result is the n-term Taylor attention of every key (Eq. (5)); only the
// base's rounding differs from the float32 state.  Per step the read kernel
// moves the bfloat16 base once (19.6 KB per head at n = 3, against 79.6 KB
// read and written for the float32 state), the window tokens and T.
#include "taylor_device.h"
#include "taylor_launch.h"

namespace taylor {
namespace lp {

__constant__ FeatureTable kTab = make_feature_table();

constexpr int kThreads = 256;
constexpr int kRG = 32;       // row groups: 8 threads per row, 8 value columns each
constexpr int kMaxWin = 128;  // window tokens (4 per row group)

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t pack_bf(float lo, float hi) {
  const bf16x2 p = {f32_to_bf16(lo), f32_to_bf16(hi)};
  return __builtin_bit_cast(uint32_t, p);
}

template <typename T> __device__ __forceinline__ void load8(const T* p, float (&x)[8]);
template <> __device__ __forceinline__ void load8<float>(const float* p, float (&x)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
template <> __device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&x)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf_lo(w[i]);
    x[2 * i + 1] = bf_hi(w[i]);
  }
}

// p_n(y) = sum_{m<n} y^m / m! by Horner's rule.
template <int NT>
__device__ __forceinline__ float poly(float y) {
  float w = 1.0f;
#pragma unroll
  for (int m = NT - 1; m >= 1; --m) w = 1.0f + w * y * (1.0f / (float)m);
  return w;
}

// Reduction of the threads' partial reads (thread (rg, cc) holds columns
// 8cc..8cc+7 summed over its rows and window tokens) and o = y[:d_v] / y[d_v].
template <typename TOUT>
__device__ __forceinline__ void finish(float (&acc)[8], float dacc, TOUT* __restrict__ o, int bh, int tid) {
  __shared__ __align__(16) float red[4][kDV];
  __shared__ float red_den[4];
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int off = 8; off <= 32; off <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += __shfl_xor(acc[i], off);
#pragma unroll
  for (int off = 1; off <= 32; off <<= 1) dacc += __shfl_xor(dacc, off);
  if (lane < 8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) red[wave][8 * lane + i] = acc[i];
  }
  if (lane == 0) red_den[wave] = dacc;
  __syncthreads();
  if (tid < kDV) {
    const float y = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
    const float den = red_den[0] + red_den[1] + red_den[2] + red_den[3];
    Elem<TOUT>::store(o, (size_t)bh * kDV + tid, y / den);
  }
}

// One step: append the token to the window at slot `step`, then
// o = (phi_hat(q) [S | T] + sum_{j <= step} p_n(q.k_j / a) [v_j; 1])[:d_v] / (...)[d_v].
template <int NT, typename TIN, typename TOUT>
__global__ __launch_bounds__(kThreads) void read_kernel(const TIN* __restrict__ q, const TIN* __restrict__ k,
                                                        const TIN* __restrict__ v, TOUT* __restrict__ o,
                                                        const uint16_t* __restrict__ S, const float* __restrict__ T,
                                                        TIN* __restrict__ wk, TIN* __restrict__ wv, int step,
                                                        int window, float inv_a) {
  constexpr int D = state_width(NT);
  constexpr int kRows = (D + kRG - 1) / kRG;
  const int bh = blockIdx.x, tid = threadIdx.x, rg = tid >> 3, cc = tid & 7;
  const uint16_t* __restrict__ Sh = S + (size_t)bh * D * kDV;
  const TIN* __restrict__ wkh = wk + (size_t)bh * window * kD;
  const TIN* __restrict__ wvh = wv + (size_t)bh * window * kDV;

  // loads first: the new token's q, k, v (one element per thread), this
  // thread's rows of the base (8 bfloat16 each; rows past D clamped), its T
  // entry, and the earlier window tokens it handles (j = rg + 32u < step)
  float xin = 0.f;
  if (tid < kD) xin = Elem<TIN>::load(q, (size_t)bh * kD + tid);
  else if (tid < 2 * kD) xin = Elem<TIN>::load(k, (size_t)bh * kD + tid - kD);
  else if (tid < 2 * kD + kDV) xin = Elem<TIN>::load(v, (size_t)bh * kDV + tid - 2 * kD);
  uint4 sv[kRows];
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int r = min(rg + kRG * i, D - 1);
    sv[i] = *reinterpret_cast<const uint4*>(Sh + (size_t)r * kDV + 8 * cc);
  }
  const float tv = T[(size_t)bh * D + min(tid, D - 1)];
  constexpr int kU = kMaxWin / kRG;
  float kw[kU][kD], vw[kU][8];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int j = min(rg + kRG * u, max(step - 1, 0));
#pragma unroll
    for (int e = 0; e < kD; e += 8) {
      float x8[8];
      load8<TIN>(wkh + (size_t)j * kD + e, x8);
#pragma unroll
      for (int i = 0; i < 8; ++i) kw[u][e + i] = x8[i];
    }
    load8<TIN>(wvh + (size_t)j * kDV + 8 * cc, vw[u]);
  }

  __shared__ float xq[kD], xk[kD];
  __shared__ __align__(16) float xv[kDV];
  __shared__ float phq[D];
  if (tid < kD) xq[tid] = xin;
  else if (tid < 2 * kD) xk[tid - kD] = xin;
  else if (tid < 2 * kD + kDV) xv[tid - 2 * kD] = xin;
  __syncthreads();
  // the new token goes into the window (read back only by later calls)
  if (tid >= kD && tid < 2 * kD) Elem<TIN>::store(wk, ((size_t)bh * window + step) * kD + tid - kD, xin);
  else if (tid >= 2 * kD && tid < 2 * kD + kDV)
    Elem<TIN>::store(wv, ((size_t)bh * window + step) * kDV + tid - 2 * kD, xin);
  const float a2 = inv_a * inv_a;
  const float4 alpha_q = make_float4(1.0f, inv_a, 0.5f * a2, 0.0f);
  if (tid < D) phq[tid] = feature_value(kTab, tid, xq, alpha_q);
  __syncthreads();

  // state part: the base rows (bfloat16 -> float32, exact) and T
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int r = rg + kRG * i;
    if (r < D) {
      const float pq = phq[r];
      const uint32_t w4[4] = {sv[i].x, sv[i].y, sv[i].z, sv[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += pq * bf_lo(w4[e]);
        acc[2 * e + 1] += pq * bf_hi(w4[e]);
      }
    }
  }
  float dacc = tid < D ? phq[tid] * tv : 0.0f;
  // window part: keys j < step from the window, key `step` (the new token)
  // from LDS; weight p_n(q.k_j / a), the same for the value columns and the
  // normaliser (counted once per row group, by cc == 0)
  float qv[kD];
#pragma unroll
  for (int e = 0; e < kD; ++e) qv[e] = xq[e] * inv_a;
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int j = rg + kRG * u;
    if (j < step) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < kD; ++e) s += qv[e] * kw[u][e];
      const float w = poly<NT>(s);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += w * vw[u][i];
      if (cc == 0) dacc += w;
    }
  }
  if (rg == (step & (kRG - 1))) {  // the new token, by one row group
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < kD; ++e) s += qv[e] * xk[e];
    const float w = poly<NT>(s);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += w * xv[8 * cc + i];
    if (cc == 0) dacc += w;
  }
  finish<TOUT>(acc, dacc, o, bh, tid);
}

// The fold: S <- round_bf16(S + sum_{j<K} phi(k_j) v_j^T), T <- T + sum_j phi(k_j).
// The S increment is the product phi(K_w)^T V_w (D x K times K x d_v) on the
// float32 matrix cores (16x16x4): wave w accumulates the 16-row feature tiles
// w, w + 4, w + 8 against the four 16-column tiles; the A operand (feature of
// row 16 ft + li for token 4s + g) is formed from the staged keys as it is
// needed, and the same features summed over the tokens give T's increment.
// The head's bfloat16 rows of S are loaded as 16-byte units before anything
// else, so they arrive while the products run; the increment goes through
// LDS (where the window was) so that every thread adds, rounds and stores
// whole 16-byte units.  Each element of S is rounded once.
template <int NT, typename TIN>
__global__ __launch_bounds__(kThreads) void fold_kernel(uint16_t* __restrict__ S, float* __restrict__ T,
                                                        const TIN* __restrict__ wk, const TIN* __restrict__ wv,
                                                        int window) {
  constexpr int D = state_width(NT);
  constexpr int NFT = (D + 15) / 16;                     // 16-row feature tiles
  constexpr int TPW = (NFT + 3) / 4;                     // tiles per wave (at most)
  constexpr int NU = (D * 8 + kThreads - 1) / kThreads;  // 16-byte units of S per thread
  constexpr int kIS = kDV + 4;                           // row stride of the staged increment
  constexpr int kLds = kMaxWin * (kD + 1) + kMaxWin * (kDV + 4);
  static_assert(D * kIS <= kLds, "the increment fits where the window was staged");
  __shared__ __align__(16) float lds[kLds];
  float(*ks)[kD + 1] = reinterpret_cast<float(*)[kD + 1]>(lds);
  float(*vs)[kDV + 4] = reinterpret_cast<float(*)[kDV + 4]>(lds + kMaxWin * (kD + 1));
  float* inc = lds;  // [D][kIS], after the products
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint16_t* __restrict__ Sh = S + (size_t)bh * D * kDV;
  uint4 sv[NU];  // units tid, tid + kThreads, ... of the head's S (8 bfloat16 each)
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int e = tid + kThreads * u;
    sv[u] = e < D * 8 ? *reinterpret_cast<const uint4*>(Sh + (size_t)e * 8) : make_uint4(0u, 0u, 0u, 0u);
  }
  const int kpad = (window + 3) & ~3;  // whole k-steps of 4 tokens; padding tokens are zero
  for (int i = tid; i < kpad * kD; i += kThreads) {
    const int j = i / kD;
    ks[j][i % kD] = j < window ? Elem<TIN>::load(wk, (size_t)bh * window * kD + i) : 0.0f;
  }
  for (int i = tid; i < kpad * kDV; i += kThreads) {
    const int j = i / kDV;
    vs[j][i % kDV] = j < window ? Elem<TIN>::load(wv, (size_t)bh * window * kDV + i) : 0.0f;
  }
  __syncthreads();
  const float4 ones = make_float4(1.f, 1.f, 1.f, 1.f);
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[TPW][4];
  float tsum[TPW];
  uint32_t code[TPW];
  float wt[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int r = min(16 * (w + 4 * i) + li, D - 1);
    code[i] = kTab.code[r];
    wt[i] = 16 * (w + 4 * i) + li < D ? kTab.weight[r] : 0.0f;  // rows past D contribute nothing
    tsum[i] = 0.0f;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[i][ct] = zero;
  }
  for (int s4 = 0; s4 < kpad; s4 += 4) {
    const int j = s4 + g;  // token of this lane's k-slot
    float bv[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) bv[ct] = vs[j][16 * ct + li];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      if (w + 4 * i < NFT) {  // uniform
        const float f = feature_value(code[i], wt[i], ks[j], ones);
        tsum[i] += j < window ? f : 0.0f;  // padding tokens have phi_0 = 1: not counted in T
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[i][ct] = mfma_f32_k4(f, bv[ct], acc[i][ct]);
      }
    }
  }
  // T of row 16 ft + li: the lane's tokens, then the other lane groups' (xor 16, 32)
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    float ts = tsum[i];
    ts += __shfl_xor(ts, 16);
    ts += __shfl_xor(ts, 32);
    const int row = 16 * (w + 4 * i) + li;
    if (w + 4 * i < NFT && g == 0 && row < D) T[(size_t)bh * D + row] += ts;
  }
  __syncthreads();  // every wave is done with the staged window
  // lane (li, g) holds rows 16 ft + 4g + r, column 16 ct + li of the increment
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    if (w + 4 * i >= NFT) continue;  // uniform
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * (w + 4 * i) + 4 * g + r;
      if (row < D) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) inc[row * kIS + 16 * ct + li] = acc[i][ct][r];
      }
    }
  }
  __syncthreads();
  // add and round, 8 values (one 16-byte unit) at a time
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int e = tid + kThreads * u;
    if (e < D * 8) {
      const float* x = inc + (e >> 3) * kIS + (e & 7) * 8;
      const float4 a0 = *reinterpret_cast<const float4*>(x), a1 = *reinterpret_cast<const float4*>(x + 4);
      uint4 o;
      o.x = pack_bf(bf_lo(sv[u].x) + a0.x, bf_hi(sv[u].x) + a0.y);
      o.y = pack_bf(bf_lo(sv[u].y) + a0.z, bf_hi(sv[u].y) + a0.w);
      o.z = pack_bf(bf_lo(sv[u].z) + a1.x, bf_hi(sv[u].z) + a1.y);
      o.w = pack_bf(bf_lo(sv[u].w) + a1.z, bf_hi(sv[u].w) + a1.w);
      *reinterpret_cast<uint4*>(Sh + (size_t)e * 8) = o;
    }
  }
}

__global__ __launch_bounds__(256) void to_bf16_kernel(const float* __restrict__ src_S, const float* __restrict__ src_T,
                                                      uint16_t* __restrict__ S, float* __restrict__ T, size_t ns,
                                                      size_t nt) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < ns; i += stride)
    S[i] = __builtin_bit_cast(uint16_t, f32_to_bf16(src_S[i]));
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < nt; i += stride) T[i] = src_T[i];
}

template <int NT, typename TIN, typename TOUT>
hipError_t launch_t(const Bf16DecodeArgs& a) {
  constexpr int D = state_width(NT);
  uint16_t* S = static_cast<uint16_t*>(a.state);
  float* T = reinterpret_cast<float*>(S + (size_t)a.BH * D * kDV);
  hipLaunchKernelGGL((read_kernel<NT, TIN, TOUT>), dim3(a.BH), dim3(kThreads), 0, a.stream,
                     static_cast<const TIN*>(a.q), static_cast<const TIN*>(a.k), static_cast<const TIN*>(a.v),
                     static_cast<TOUT*>(a.o), S, T, static_cast<TIN*>(a.win_k), static_cast<TIN*>(a.win_v), a.step,
                     a.window, 1.0f / a.a);
  if (a.step == a.window - 1)
    hipLaunchKernelGGL((fold_kernel<NT, TIN>), dim3(a.BH), dim3(kThreads), 0, a.stream, S, T,
                       static_cast<const TIN*>(a.win_k), static_cast<const TIN*>(a.win_v), a.window);
  return hipGetLastError();
}

template <int NT>
hipError_t launch_n(const Bf16DecodeArgs& a) {
  if (a.in_bf16) return a.out_bf16 ? launch_t<NT, uint16_t, uint16_t>(a) : launch_t<NT, uint16_t, float>(a);
  return a.out_bf16 ? launch_t<NT, float, uint16_t>(a) : launch_t<NT, float, float>(a);
}

}  // namespace lp

int bf16_decode_max_window() { return lp::kMaxWin; }

hipError_t launch_decode_bf16state(const Bf16DecodeArgs& a) {
  switch (a.n) {
    case 1: return lp::launch_n<1>(a);
    case 2: return lp::launch_n<2>(a);
    case 3: return lp::launch_n<3>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_state_to_bf16(const float* state, void* state_bf16, int BH, int D, hipStream_t stream) {
  const size_t ns = (size_t)BH * D * kDV, nt = (size_t)BH * D;
  if (ns == 0) return hipSuccess;
  uint16_t* S = static_cast<uint16_t*>(state_bf16);
  float* T = reinterpret_cast<float*>(S + ns);
  const size_t blocks = (ns + 255) / 256;
  hipLaunchKernelGGL(lp::to_bf16_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0, stream, state,
                     state + ns, S, T, ns, nt);
  return hipGetLastError();
}

}  // namespace taylor
