// Chunked prefill (section 3.5 of "A Taylor-Series Route to Linear-Time
// Transformers with a Fixed Number of Recurrent States", arXiv 2610.20637).
//
// For every head the sequence is cut into chunks of C tokens.  Chunk j's
// outputs are
//     Y = phi_hat(Q_j) A_{<j}  +  tril(p_n(Q_j K_j^T / a)) [V_j, 1]
//     o = Y[:, :d_v] / Y[:, d_v]
// (the off-diagonal part through the states, Eq. (5); the masked c x c block on
// the diagonal, Eq. (1)-(2)), after which the state takes the chunk:
//     A_{<j+1} = A_{<j} + phi(K_j)^T [V_j, 1]                (Eq. (6)-(7) summed).
// States are additive (section 5.2), so the chunks of one head are split into
// segments that run on different workgroups:
//   1. segment sums  : A_seg = sum over the segment's chunks of phi(K)^T [V, 1]
//   2. scan          : exclusive prefix of the segment sums, starting from the
//                      caller's state
//   3. chunk kernel  : each segment replays its chunks from its prefix.
//
// Layout of the work inside one 256-thread workgroup (4 waves):
//   - the S part of the state (D x 64, float32) lives in MFMA accumulator
//     registers for the whole segment: wave w owns value columns 16w..16w+15,
//     a 16-row tile of S is one f32x4 per lane (rows 4*(lane/16)+r, column
//     lane%16);
//   - the ones-column T (D floats) lives in LDS;
//   - per chunk, q/k (as float), v, phi_hat(Q), phi(K) and the masked
//     polynomial block P are staged in LDS; every contraction is an MFMA
//     (bfloat16 16x16x32 with float32 accumulation for bfloat16 inputs,
//     float32 16x16x4 for float32 inputs).
//   - the state is read straight from the accumulators: for a bfloat16 read the
//     two 16-row tiles of one 32-feature block are packed into one B operand,
//     and the query features are fetched in the matching k-slot order.
#include <type_traits>

#include "taylor_device.h"
#include "taylor_launch.h"

namespace taylor {

template <int NT, bool BF, int C>
struct PrefillShape {
  static constexpr int D = state_width(NT);
  static constexpr int DP = round_up(D, 32);  // padded feature count
  static constexpr int NFT = DP / 16;         // 16-row feature tiles
  static constexpr int NTT = C / 16;          // 16-token tiles per chunk
  // LDS row strides in elements (padding keeps the hot reads bank-spread and
  // the vector accesses aligned).
  static constexpr int QS = BF ? DP + 4 : DP + 1;     // PhQ [C][QS]
  static constexpr int KS = BF ? C + 8 : DP + 16;     // BF: PhK^T [DP][KS]; F32: PhK [C][KS]
  static constexpr int VS = BF ? C + 8 : kDV + 16;    // BF: V^T [64][VS];   F32: V [C][VS]
  static constexpr int PS = BF ? C + 8 : C + 1;       // P [C][PS]
};

// p_n(y) = sum_{m<n} y^m / m!  (Horner), y = q.k / a.
template <int NT>
__device__ __forceinline__ float taylor_poly(float y) {
  float w = 1.0f;
#pragma unroll
  for (int m = NT - 1; m >= 1; --m) w = 1.0f + w * y * (1.0f / (float)m);
  return w;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 p = {f32_to_bf16(lo), f32_to_bf16(hi)};
  return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

template <int NT, bool BF, int C, bool FULL, typename TOUT>
__global__ __launch_bounds__(256) void prefill_chunk_kernel(
    const void* __restrict__ q_, const void* __restrict__ k_, const void* __restrict__ v_,
    TOUT* __restrict__ o,
    const float* __restrict__ pre_S, const float* __restrict__ pre_T, int pre_slots,
    float* __restrict__ dst_S, float* __restrict__ dst_T, int dst_slots,
    int N, int nseg, int cps, float inv_a) {
  using Sh = PrefillShape<NT, BF, C>;
  constexpr int D = Sh::D, DP = Sh::DP, NFT = Sh::NFT, NTT = Sh::NTT;
  using LT = std::conditional_t<BF, uint16_t, float>;  // LDS element of phi, P, V
  using IT = std::conditional_t<BF, uint16_t, float>;  // global input element

  const IT* __restrict__ q = static_cast<const IT*>(q_);
  const IT* __restrict__ k = static_cast<const IT*>(k_);
  const IT* __restrict__ v = static_cast<const IT*>(v_);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, g = lane >> 4;
  const int gseg = FULL ? nseg : nseg - 1;
  const int bh = blockIdx.x / gseg, seg = blockIdx.x % gseg;
  const int t_begin = seg * cps * C;
  const int t_end = min(N, t_begin + cps * C);
  const int col = 16 * w + li;  // value column owned by this lane

  __shared__ __align__(16) float Xq[FULL ? C : 1][kD];
  __shared__ __align__(16) float Xk[C][kD];
  __shared__ __align__(16) LT PhQ[FULL ? C : 1][Sh::QS];
  __shared__ __align__(16) LT PhK[BF ? DP : C][Sh::KS];
  __shared__ __align__(16) LT Vl[BF ? kDV : C][Sh::VS];
  __shared__ __align__(16) LT P[FULL ? C : 1][Sh::PS];
  __shared__ float Ts[DP];
  __shared__ float den[FULL ? C : 1];

  // ---- the segment's starting state -------------------------------------
  f32x4 Sacc[NFT];
  {
    const float* ps = pre_S ? pre_S + ((size_t)bh * pre_slots + (pre_slots == 1 ? 0 : seg)) * D * kDV : nullptr;
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * ft + 4 * g + r;
        Sacc[ft][r] = (ps && row < D) ? ps[(size_t)row * kDV + col] : 0.0f;
      }
    if (tid < DP) {
      const float* pt = pre_T ? pre_T + ((size_t)bh * pre_slots + (pre_slots == 1 ? 0 : seg)) * D : nullptr;
      Ts[tid] = (pt && tid < D) ? pt[tid] : 0.0f;
    }
  }

  const float a2 = inv_a * inv_a;
  const float am_q[3] = {1.0f, inv_a, 0.5f * a2};
  const float am_k[3] = {1.0f, 1.0f, 1.0f};

  for (int t0 = t_begin; t0 < t_end; t0 += C) {
    const int nv = min(C, t_end - t0);
    const size_t tok0 = (size_t)bh * N + t0;

    // ---- phase 1: stage q, k (as float) and v ----------------------------
    if constexpr (BF) {
      constexpr int NQK = FULL ? 4 * C : 2 * C;  // 16-byte loads of q and k
      for (int i = tid; i < NQK; i += 256) {
        const bool isk = FULL ? (i >= 2 * C) : true;
        const int rem = (FULL && isk) ? i - 2 * C : i;
        const int tok = rem >> 1, half = rem & 1;
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (tok < nv) raw = *reinterpret_cast<const uint4*>((isk ? k : q) + (tok0 + tok) * kD + 8 * half);
        float* dst = isk ? &Xk[tok][8 * half] : &Xq[FULL ? tok : 0][8 * half];
        *reinterpret_cast<float4*>(dst) = make_float4(bf16_lo(raw.x), bf16_hi(raw.x), bf16_lo(raw.y), bf16_hi(raw.y));
        *reinterpret_cast<float4*>(dst + 4) = make_float4(bf16_lo(raw.z), bf16_hi(raw.z), bf16_lo(raw.w), bf16_hi(raw.w));
      }
      for (int i = tid; i < 8 * C; i += 256) {  // v -> V^T
        const int tok = i >> 3, c8 = i & 7;
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (tok < nv) raw = *reinterpret_cast<const uint4*>(v + (tok0 + tok) * kDV + 8 * c8);
        const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          Vl[8 * c8 + 2 * j][tok] = (uint16_t)(wd[j] & 0xFFFFu);
          Vl[8 * c8 + 2 * j + 1][tok] = (uint16_t)(wd[j] >> 16);
        }
      }
    } else {
      constexpr int NQK = FULL ? 8 * C : 4 * C;  // float4 loads of q and k
      for (int i = tid; i < NQK; i += 256) {
        const bool isk = FULL ? (i >= 4 * C) : true;
        const int rem = (FULL && isk) ? i - 4 * C : i;
        const int tok = rem >> 2, qu = rem & 3;
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (tok < nv) x = *reinterpret_cast<const float4*>((isk ? k : q) + (tok0 + tok) * kD + 4 * qu);
        float* dst = isk ? &Xk[tok][4 * qu] : &Xq[FULL ? tok : 0][4 * qu];
        *reinterpret_cast<float4*>(dst) = x;
      }
      for (int i = tid; i < 16 * C; i += 256) {
        const int tok = i >> 4, c4 = i & 15;
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (tok < nv) x = *reinterpret_cast<const float4*>(v + (tok0 + tok) * kDV + 4 * c4);
        *reinterpret_cast<float4*>(&Vl[tok][4 * c4]) = x;
      }
    }
    __syncthreads();

    // ---- phase 2: feature maps phi_hat(Q) and phi(K) ---------------------
    {
      auto phi_rows = [&](auto isq_c, auto f0_c, auto f1_c) {
        constexpr bool ISQ = decltype(isq_c)::value;
        constexpr int F0 = decltype(f0_c)::value, F1 = decltype(f1_c)::value;
        for (int tok = lane; tok < C; tok += 64) {
          float x[kD];
          const float* src = ISQ ? &Xq[FULL ? tok : 0][0] : &Xk[tok][0];
#pragma unroll
          for (int j = 0; j < kD; j += 4) {
            const float4 t = *reinterpret_cast<const float4*>(src + j);
            x[j] = t.x; x[j + 1] = t.y; x[j + 2] = t.z; x[j + 3] = t.w;
          }
          float vals[F1 - F0];
          for_features<NT, F0, F1>(x, ISQ ? am_q : am_k, [&](int f, float val) { vals[f] = val; });
          if constexpr (ISQ) {
            if constexpr (BF) {
#pragma unroll
              for (int f = 0; f < F1 - F0; f += 4) {
                const uint2 pk = make_uint2(pack_bf16x2(vals[f], vals[f + 1]), pack_bf16x2(vals[f + 2], vals[f + 3]));
                *reinterpret_cast<uint2*>(&PhQ[FULL ? tok : 0][F0 + f]) = pk;
              }
            } else {
#pragma unroll
              for (int f = 0; f < F1 - F0; ++f) PhQ[FULL ? tok : 0][F0 + f] = vals[f];
            }
          } else {
            const bool valid = tok < nv;  // padding tokens must not reach the state
#pragma unroll
            for (int f = 0; f < F1 - F0; ++f) {
              const float val = valid ? vals[f] : 0.0f;
              if constexpr (BF) {
                PhK[F0 + f][tok] = __builtin_bit_cast(uint16_t, f32_to_bf16(val));
              } else {
                PhK[tok][F0 + f] = val;
              }
            }
          }
        }
      };
      using T_ = std::true_type;
      using F_ = std::false_type;
      if constexpr (FULL) {
        constexpr int H = round_up(DP / 2, 4);
        if (w == 0) phi_rows(T_{}, std::integral_constant<int, 0>{}, std::integral_constant<int, H>{});
        else if (w == 1) phi_rows(T_{}, std::integral_constant<int, H>{}, std::integral_constant<int, DP>{});
        else if (w == 2) phi_rows(F_{}, std::integral_constant<int, 0>{}, std::integral_constant<int, H>{});
        else phi_rows(F_{}, std::integral_constant<int, H>{}, std::integral_constant<int, DP>{});
      } else {
        constexpr int Q4 = DP / 4;
        if (w == 0) phi_rows(F_{}, std::integral_constant<int, 0>{}, std::integral_constant<int, Q4>{});
        else if (w == 1) phi_rows(F_{}, std::integral_constant<int, Q4>{}, std::integral_constant<int, 2 * Q4>{});
        else if (w == 2) phi_rows(F_{}, std::integral_constant<int, 2 * Q4>{}, std::integral_constant<int, 3 * Q4>{});
        else phi_rows(F_{}, std::integral_constant<int, 3 * Q4>{}, std::integral_constant<int, DP>{});
      }
    }
    __syncthreads();

    if constexpr (FULL) {
      // ---- phase 3: masked polynomial block P and the normaliser ----------
      for (int tt = w; tt < NTT; tt += 4) {
        const int tok = 16 * tt + li;
        float dsum = 0.0f;
        const int ktmax = min(tt | 1, NTT - 1);
        for (int kt = 0; kt <= ktmax; ++kt) {
          float p[4] = {0.f, 0.f, 0.f, 0.f};
          if (kt <= tt) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
            if constexpr (BF) {
              const float4 xk = *reinterpret_cast<const float4*>(&Xk[16 * kt + li][4 * g]);
              const float4 xq = *reinterpret_cast<const float4*>(&Xq[tok][4 * g]);
              const bf16x4 ak = {f32_to_bf16(xk.x), f32_to_bf16(xk.y), f32_to_bf16(xk.z), f32_to_bf16(xk.w)};
              const bf16x4 bq = {f32_to_bf16(xq.x), f32_to_bf16(xq.y), f32_to_bf16(xq.z), f32_to_bf16(xq.w)};
              s = mfma_bf16_k16(ak, bq, s);
            } else {
#pragma unroll
              for (int st = 0; st < 4; ++st) s = mfma_f32_k4(Xk[16 * kt + li][4 * st + g], Xq[tok][4 * st + g], s);
            }
            // lane holds S(token = tok, key = 16kt + 4g + r)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = 16 * kt + 4 * g + r;
              p[r] = key <= tok ? taylor_poly<NT>(s[r] * inv_a) : 0.0f;
            }
          }
          if constexpr (BF) {
            const uint32_t lo = pack_bf16x2(p[0], p[1]), hi = pack_bf16x2(p[2], p[3]);
            dsum += bf16_lo(lo) + bf16_hi(lo) + bf16_lo(hi) + bf16_hi(hi);
            *reinterpret_cast<uint2*>(&P[tok][16 * kt + 4 * g]) = make_uint2(lo, hi);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              dsum += p[r];
              P[tok][16 * kt + 4 * g + r] = p[r];
            }
          }
        }
        // off-diagonal part of the normaliser: phi_hat(q_t) . T
        float part = 0.0f;
        constexpr int FQ = DP / 4;
        if constexpr (BF) {
#pragma unroll
          for (int f = 0; f < FQ; f += 4) {
            const uint2 u = *reinterpret_cast<const uint2*>(&PhQ[tok][g * FQ + f]);
            part += bf16_lo(u.x) * Ts[g * FQ + f] + bf16_hi(u.x) * Ts[g * FQ + f + 1] +
                    bf16_lo(u.y) * Ts[g * FQ + f + 2] + bf16_hi(u.y) * Ts[g * FQ + f + 3];
          }
        } else {
#pragma unroll
          for (int f = 0; f < FQ; ++f) part += PhQ[tok][g * FQ + f] * Ts[g * FQ + f];
        }
        float tot = dsum + part;
        tot += __shfl_xor(tot, 16);
        tot += __shfl_xor(tot, 32);
        if (g == 0) den[tok] = tot;
      }
      __syncthreads();

      // ---- phase 4: Y = phi_hat(Q) S + P V, then o = Y / den -------------
      if constexpr (BF) {
        bf16x8 bs[NFT / 2];
#pragma unroll
        for (int kb = 0; kb < NFT / 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            bs[kb][r] = f32_to_bf16(Sacc[2 * kb][r]);
            bs[kb][4 + r] = f32_to_bf16(Sacc[2 * kb + 1][r]);
          }
        for (int mt = 0; mt < NTT; ++mt) {
          const int tok = 16 * mt + li;
          f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < NFT / 2; ++kb) {
            const uint2 lo = *reinterpret_cast<const uint2*>(&PhQ[tok][32 * kb + 4 * g]);
            const uint2 hi = *reinterpret_cast<const uint2*>(&PhQ[tok][32 * kb + 16 + 4 * g]);
            const uint4 a4 = make_uint4(lo.x, lo.y, hi.x, hi.y);
            y = mfma_bf16_k32(__builtin_bit_cast(bf16x8, a4), bs[kb], y);
          }
          const int nkb = (16 * mt + 15) / 32 + 1;
          for (int kb = 0; kb < nkb; ++kb) {
            const uint4 a4 = *reinterpret_cast<const uint4*>(&P[tok][32 * kb + 8 * g]);
            const uint4 b4 = *reinterpret_cast<const uint4*>(&Vl[col][32 * kb + 8 * g]);
            y = mfma_bf16_k32(__builtin_bit_cast(bf16x8, a4), __builtin_bit_cast(bf16x8, b4), y);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 16 * mt + 4 * g + r;
            if (row < nv) Elem<TOUT>::store(o, (tok0 + row) * kDV + col, y[r] / den[row]);
          }
        }
      } else {
        for (int mt = 0; mt < NTT; ++mt) {
          const int tok = 16 * mt + li;
          f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
            for (int r = 0; r < 4; ++r) y = mfma_f32_k4(PhQ[tok][16 * ft + 4 * g + r], Sacc[ft][r], y);
          const int nst = (16 * mt + 16) / 4;
          for (int st = 0; st < nst; ++st) y = mfma_f32_k4(P[tok][4 * st + g], Vl[4 * st + g][col], y);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 16 * mt + 4 * g + r;
            if (row < nv) Elem<TOUT>::store(o, (tok0 + row) * kDV + col, y[r] / den[row]);
          }
        }
      }
    }

    // ---- phase 5: A += phi(K)^T [V, 1] -------------------------------------
    if constexpr (BF) {
#pragma unroll
      for (int kb = 0; kb < C / 32; ++kb) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&Vl[col][32 * kb + 8 * g]));
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&PhK[16 * ft + li][32 * kb + 8 * g]));
          Sacc[ft] = mfma_bf16_k32(a, b, Sacc[ft]);
        }
      }
      if (tid < DP) {
        float s = 0.0f;
#pragma unroll
        for (int t = 0; t < C; t += 8) {
          const uint4 u = *reinterpret_cast<const uint4*>(&PhK[tid][t]);
          s += bf16_lo(u.x) + bf16_hi(u.x) + bf16_lo(u.y) + bf16_hi(u.y) + bf16_lo(u.z) + bf16_hi(u.z) +
               bf16_lo(u.w) + bf16_hi(u.w);
        }
        Ts[tid] += s;
      }
    } else {
      for (int st = 0; st < C / 4; ++st) {
        const float b = Vl[4 * st + g][col];
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) Sacc[ft] = mfma_f32_k4(PhK[4 * st + g][16 * ft + li], b, Sacc[ft]);
      }
      if (tid < DP) {
        float s = 0.0f;
        for (int t = 0; t < C; ++t) s += PhK[t][tid];
        Ts[tid] += s;
      }
    }
    __syncthreads();
  }

  // ---- write the state out -------------------------------------------------
  const bool write = FULL ? (seg == nseg - 1) : true;
  if (write) {
    const size_t slot = (size_t)bh * dst_slots + (dst_slots == 1 ? 0 : seg);
    float* ds = dst_S + slot * D * kDV;
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * ft + 4 * g + r;
        if (row < D) ds[(size_t)row * kDV + col] = Sacc[ft][r];
      }
    if (tid < D) dst_T[slot * D + tid] = Ts[tid];
  }
}

// Exclusive scan of the segment sums, in place, seeded with the caller's state:
// slot s <- state + sum_{s' < s} (segment sum s').  Slot nseg-1 never holds a
// sum (the last segment's total is not needed), only its prefix.
__global__ __launch_bounds__(256) void segment_scan_kernel(const float* __restrict__ st_S,
                                                           const float* __restrict__ st_T,
                                                           float* __restrict__ W_S, float* __restrict__ W_T,
                                                           int D, int nseg) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int nS = D * kDV;
  if (e >= nS + D) return;
  const float* src;
  float* slot0;
  size_t stride;
  if (e < nS) {
    src = st_S + (size_t)bh * nS + e;
    slot0 = W_S + (size_t)bh * nseg * nS + e;
    stride = nS;
  } else {
    src = st_T + (size_t)bh * D + (e - nS);
    slot0 = W_T + (size_t)bh * nseg * D + (e - nS);
    stride = D;
  }
  float run = *src;
  for (int s = 0; s < nseg; ++s) {
    float* p = slot0 + (size_t)s * stride;
    const float tmp = (s < nseg - 1) ? *p : 0.0f;
    *p = run;
    run += tmp;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
PrefillPlan plan_prefill(int BH, int N, int n, int chunk) {
  PrefillPlan p;
  if (BH <= 0 || N <= 0 || chunk <= 0) return p;
  p.nchunks = (N + chunk - 1) / chunk;
  // Aim for at least 512 workgroups in the chunk kernel (two per CU on a
  // 256-CU part) when the heads alone do not provide them.
  int nseg = (512 + BH - 1) / BH;
  if (nseg < 1) nseg = 1;
  if (nseg > p.nchunks) nseg = p.nchunks;
  p.chunks_per_seg = (p.nchunks + nseg - 1) / nseg;
  p.nseg = (p.nchunks + p.chunks_per_seg - 1) / p.chunks_per_seg;
  const int D = n == 1 ? state_width(1) : n == 2 ? state_width(2) : n == 3 ? state_width(3) : state_width(4);
  p.workspace_floats = p.nseg > 1 ? (size_t)BH * p.nseg * D * (kDV + 1) : 0;
  return p;
}

bool prefill_supported(int n, int chunk, bool in_bf16) {
  if (n < 1 || n > 3) return false;
  if (in_bf16) return chunk == 32 || chunk == 64 || chunk == 128;
  return chunk == 32 || chunk == 64;
}

template <int NT, bool BF, int C, typename TOUT>
static hipError_t launch_prefill_t(const PrefillArgs& a) {
  constexpr int D = state_width(NT);
  const PrefillPlan& pl = a.plan;
  float* st_S = a.state;
  float* st_T = a.state + (size_t)a.BH * D * kDV;
  const float inv_a = 1.0f / a.a;
  hipEvent_t* ev = a.events;
  if (ev) (void)hipEventRecord(ev[0], a.stream);
  if (pl.nseg > 1) {
    float* W_S = a.workspace;
    float* W_T = a.workspace + (size_t)a.BH * pl.nseg * D * kDV;
    hipLaunchKernelGGL((prefill_chunk_kernel<NT, BF, C, false, TOUT>), dim3(a.BH * (pl.nseg - 1)), dim3(256), 0,
                       a.stream, a.q, a.k, a.v, static_cast<TOUT*>(nullptr), (const float*)nullptr,
                       (const float*)nullptr, 1, W_S, W_T, pl.nseg, a.N, pl.nseg, pl.chunks_per_seg, inv_a);
    if (ev) (void)hipEventRecord(ev[1], a.stream);
    dim3 sgrid((D * (kDV + 1) + 255) / 256, a.BH);
    hipLaunchKernelGGL(segment_scan_kernel, sgrid, dim3(256), 0, a.stream, st_S, st_T, W_S, W_T, D, pl.nseg);
    if (ev) (void)hipEventRecord(ev[2], a.stream);
    hipLaunchKernelGGL((prefill_chunk_kernel<NT, BF, C, true, TOUT>), dim3(a.BH * pl.nseg), dim3(256), 0, a.stream,
                       a.q, a.k, a.v, static_cast<TOUT*>(a.o), W_S, W_T, pl.nseg, st_S, st_T, 1, a.N, pl.nseg,
                       pl.chunks_per_seg, inv_a);
  } else {
    if (ev) {
      (void)hipEventRecord(ev[1], a.stream);
      (void)hipEventRecord(ev[2], a.stream);
    }
    hipLaunchKernelGGL((prefill_chunk_kernel<NT, BF, C, true, TOUT>), dim3(a.BH), dim3(256), 0, a.stream, a.q, a.k,
                       a.v, static_cast<TOUT*>(a.o), st_S, st_T, 1, st_S, st_T, 1, a.N, 1, pl.chunks_per_seg,
                       inv_a);
  }
  if (ev) (void)hipEventRecord(ev[3], a.stream);
  return hipGetLastError();
}

template <int NT, bool BF, int C>
static hipError_t launch_prefill_c(const PrefillArgs& a) {
  return a.out_bf16 ? launch_prefill_t<NT, BF, C, uint16_t>(a) : launch_prefill_t<NT, BF, C, float>(a);
}

template <int NT>
static hipError_t launch_prefill_n(const PrefillArgs& a) {
  if (a.in_bf16) {
    switch (a.chunk) {
      case 32: return launch_prefill_c<NT, true, 32>(a);
      case 64: return launch_prefill_c<NT, true, 64>(a);
      case 128: return launch_prefill_c<NT, true, 128>(a);
    }
  } else {
    switch (a.chunk) {
      case 32: return launch_prefill_c<NT, false, 32>(a);
      case 64: return launch_prefill_c<NT, false, 64>(a);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs& a) {
  switch (a.n) {
    case 1: return launch_prefill_n<1>(a);
    case 2: return launch_prefill_n<2>(a);
    case 3: return launch_prefill_n<3>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace taylor
