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
// Work inside one 256-thread workgroup (4 waves of 64):
//   - the S part of the state (D x 64, float32) stays in MFMA accumulator
//     registers for the whole segment; wave w owns value columns 16w..16w+15
//     and a 16-row tile of S is one f32x4 per lane (rows 4*(lane/16)+r, column
//     lane%16).  The ones-column T is column 0 of extra accumulator tiles.
//   - global loads of chunk j+1 are issued into registers while chunk j is
//     computed (software pipelining), so HBM latency overlaps the math; the
//     outputs of chunk j are divided and stored while chunk j+1 is staged.
//   - per chunk: q, k (as float), V^T, phi_hat(Q), phi(K) and the masked
//     polynomial block P are staged in LDS and shared by the 4 waves; every
//     contraction is an MFMA (bfloat16 16x16x32 with float32 accumulation for
//     bfloat16 inputs, float32 16x16x4 for float32 inputs).
//   - the state is read straight from the accumulators: for a bfloat16 read the
//     two 16-row tiles of one 32-feature block are packed into one B operand,
//     and the query features are fetched in the matching k-slot order.  The
//     normaliser uses the same MFMAs: T (the ones-column of the state) is a
//     B column for the read (split into bfloat16 high and low parts, so it
//     keeps float32 accuracy), a ones column turns P into its row sums, and
//     the T update is phi(K)^T times a ones column, accumulated in registers.
//   - three barriers per chunk: inputs staged | features and P ready | chunk done.
#include <type_traits>

#include <algorithm>

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
  // 16-byte global loads per chunk and per thread
  static constexpr int QK_UNITS = BF ? 2 * C : 4 * C;     // units of q (and as many of k)
  static constexpr int V_UNITS = BF ? 8 * C : 16 * C;     // units of v
  static constexpr int NQK = (2 * QK_UNITS + 255) / 256;
  static constexpr int NV = (V_UNITS + 255) / 256;
  static constexpr int NTW = (NFT + 3) / 4;  // T tiles per wave (tile ft belongs to wave ft % 4)
  // two workgroups per CU when registers and LDS allow it
  static constexpr int MIN_WAVES = (BF && C <= 64) ? 2 : 1;
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
__global__ __launch_bounds__(256, (PrefillShape<NT, BF, C>::MIN_WAVES)) void prefill_chunk_kernel(
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

  // The wave index is made explicitly uniform (a scalar register): MFMA
  // instructions ignore the EXEC mask, so every condition guarding one must be
  // a scalar branch, never a per-lane predicate.
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gseg = FULL ? nseg : nseg - 1;
  const int bh = blockIdx.x / gseg, seg = blockIdx.x % gseg;
  const int t_begin = seg * cps * C;
  const int t_end = min(N, t_begin + cps * C);
  const int col = 16 * w + li;  // value column owned by this lane

  __shared__ __align__(16) float Xq[FULL ? C : 1][kD];
  __shared__ __align__(16) float Xk[C][kD];
  __shared__ __align__(16) uint16_t Xqb[(FULL && BF) ? C : 1][kD];  // raw bfloat16 q, k for Q K^T
  __shared__ __align__(16) uint16_t Xkb[BF ? C : 1][kD];
  __shared__ __align__(16) LT PhQ[FULL ? C : 1][Sh::QS];
  __shared__ __align__(16) LT PhK[BF ? DP : C][Sh::KS];
  __shared__ __align__(16) LT Vl[BF ? kDV : C][Sh::VS];
  __shared__ __align__(16) LT P[FULL ? C : 1][Sh::PS];
  // T published for the normaliser read: bfloat16 high/low parts, or float32
  __shared__ __align__(16) uint16_t Thb[(FULL && BF) ? DP : 1], Tlb[(FULL && BF) ? DP : 1];
  __shared__ __align__(16) float Ts[(FULL && !BF) ? DP : 1];
  __shared__ __align__(16) float invden[FULL ? C : 1];  // 1 / normaliser of the chunk being finished

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
  }
  // T lives in MFMA accumulators too: column 0 of tile ft (owned by wave ft % 4)
  f32x4 Tacc[Sh::NTW];
  {
    const float* pt = pre_T ? pre_T + ((size_t)bh * pre_slots + (pre_slots == 1 ? 0 : seg)) * D : nullptr;
#pragma unroll
    for (int j = 0; j < Sh::NTW; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * (w + 4 * j) + 4 * g + r;
        Tacc[j][r] = (pt && li == 0 && w + 4 * j < NFT && row < D) ? pt[row] : 0.0f;
      }
  }

  const float a2 = inv_a * inv_a;
  const float am_q[3] = {1.0f, inv_a, 0.5f * a2};

  // ---- software-pipelined global loads -------------------------------------
  // Unit i < QK_UNITS is a 16-byte piece of q, the next QK_UNITS are pieces of
  // k; v units are one token's 8 (bfloat16) or 4 (float32) consecutive columns.
  uint4 rqk[Sh::NQK], rv[Sh::NV];
  auto issue_loads = [&](int c0) {
    const int nvc = min(C, t_end - c0);
    const size_t base = (size_t)bh * N + c0;
#pragma unroll
    for (int u = 0; u < Sh::NQK; ++u) {
      const int i = tid + 256 * u;
      rqk[u] = make_uint4(0, 0, 0, 0);
      if (i < 2 * Sh::QK_UNITS) {
        const bool isk = i >= Sh::QK_UNITS;
        if (FULL || isk) {
          const int rem = isk ? i - Sh::QK_UNITS : i;
          const int tok = BF ? rem >> 1 : rem >> 2;
          const int part = BF ? rem & 1 : rem & 3;
          if (tok < nvc)
            rqk[u] = *reinterpret_cast<const uint4*>((isk ? k : q) + (base + tok) * kD + (BF ? 8 : 4) * part);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < Sh::NV; ++u) {
      const int i = tid + 256 * u;
      rv[u] = make_uint4(0, 0, 0, 0);
      if (i < Sh::V_UNITS) {
        const int tok = BF ? i >> 3 : i >> 4;
        const int part = BF ? i & 7 : i & 15;
        if (tok < nvc) rv[u] = *reinterpret_cast<const uint4*>(v + (base + tok) * kDV + (BF ? 8 : 4) * part);
      }
    }
  };
  auto stage_loads = [&]() {
#pragma unroll
    for (int u = 0; u < Sh::NQK; ++u) {
      const int i = tid + 256 * u;
      if (i < 2 * Sh::QK_UNITS) {
        const bool isk = i >= Sh::QK_UNITS;
        if (FULL || isk) {
          const int rem = isk ? i - Sh::QK_UNITS : i;
          if constexpr (BF) {
            const int tok = rem >> 1, half = rem & 1;
            float* dst = isk ? &Xk[tok][8 * half] : &Xq[FULL ? tok : 0][8 * half];
            const uint4 raw = rqk[u];
            *reinterpret_cast<uint4*>(isk ? &Xkb[tok][8 * half] : &Xqb[(FULL && BF) ? tok : 0][8 * half]) = raw;
            *reinterpret_cast<float4*>(dst) =
                make_float4(bf16_lo(raw.x), bf16_hi(raw.x), bf16_lo(raw.y), bf16_hi(raw.y));
            *reinterpret_cast<float4*>(dst + 4) =
                make_float4(bf16_lo(raw.z), bf16_hi(raw.z), bf16_lo(raw.w), bf16_hi(raw.w));
          } else {
            const int tok = rem >> 2, qu = rem & 3;
            float* dst = isk ? &Xk[tok][4 * qu] : &Xq[FULL ? tok : 0][4 * qu];
            *reinterpret_cast<uint4*>(dst) = rqk[u];
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < Sh::NV; ++u) {
      const int i = tid + 256 * u;
      if (i < Sh::V_UNITS) {
        if constexpr (BF) {  // transpose into V^T [column][token]
          const int tok = i >> 3, c8 = i & 7;
          const uint32_t wd[4] = {rv[u].x, rv[u].y, rv[u].z, rv[u].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            Vl[8 * c8 + 2 * j][tok] = (uint16_t)(wd[j] & 0xFFFFu);
            Vl[8 * c8 + 2 * j + 1][tok] = (uint16_t)(wd[j] >> 16);
          }
        } else {
          const int tok = i >> 4, c4 = i & 15;
          *reinterpret_cast<uint4*>(&Vl[tok][4 * c4]) = rv[u];
        }
      }
    }
  };
  // Publish T (held by lanes li == 0) in LDS for the normaliser read.
  auto publish_T = [&]() {
    if constexpr (FULL) {
      if (li == 0) {
#pragma unroll
        for (int j = 0; j < Sh::NTW; ++j) {
          const int ft = w + 4 * j;
          if (ft < NFT) {
            const int row = 16 * ft + 4 * g;
            if constexpr (BF) {
              float lo[4];
              uint16_t hb[4], lb[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const __bf16 h = f32_to_bf16(Tacc[j][r]);
                lo[r] = Tacc[j][r] - (float)h;
                hb[r] = __builtin_bit_cast(uint16_t, h);
                lb[r] = __builtin_bit_cast(uint16_t, f32_to_bf16(lo[r]));
              }
              *reinterpret_cast<uint2*>(&Thb[row]) =
                  make_uint2(hb[0] | (uint32_t)hb[1] << 16, hb[2] | (uint32_t)hb[3] << 16);
              *reinterpret_cast<uint2*>(&Tlb[row]) =
                  make_uint2(lb[0] | (uint32_t)lb[1] << 16, lb[2] | (uint32_t)lb[3] << 16);
            } else {
              *reinterpret_cast<float4*>(&Ts[row]) = make_float4(Tacc[j][0], Tacc[j][1], Tacc[j][2], Tacc[j][3]);
            }
          }
        }
      }
    }
  };

  f32x4 Y[NTT];  // this wave's outputs of the chunk being finished
  int prev_t0 = -1, prev_nv = 0;
  // o = Y / den for the previous chunk (den in LDS, Y in registers).
  auto epilogue = [&]() {
    if constexpr (FULL) {
      if (prev_t0 >= 0) {
        const size_t tok0 = (size_t)bh * N + prev_t0;
#pragma unroll
        for (int mt = 0; mt < NTT; ++mt) {
          const float4 inv = *reinterpret_cast<const float4*>(&invden[16 * mt + 4 * g]);
          const float iv[4] = {inv.x, inv.y, inv.z, inv.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 16 * mt + 4 * g + r;
            if (row < prev_nv) Elem<TOUT>::store(o, (tok0 + row) * kDV + col, Y[mt][r] * iv[r]);
          }
        }
      }
    }
  };

  issue_loads(t_begin);
  for (int t0 = t_begin; t0 < t_end; t0 += C) {
    const int nv = min(C, t_end - t0);

    // ---- phase 1: stage chunk j, prefetch chunk j+1, finish chunk j-1 ----
    publish_T();
    stage_loads();
    if (t0 + C < t_end) issue_loads(t0 + C);
    epilogue();
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
          // padding tokens have x = 0, so only their constant feature needs masking
          const float am_k[3] = {tok < nv ? 1.0f : 0.0f, 1.0f, 1.0f};
          float grp[4];
          for_features<NT, F0, F1>(x, ISQ ? am_q : am_k, [&](int f, float val) {
            if constexpr (ISQ) {
              grp[f & 3] = val;
              if ((f & 3) == 3) {
                if constexpr (BF) {
                  *reinterpret_cast<uint2*>(&PhQ[FULL ? tok : 0][F0 + f - 3]) =
                      make_uint2(pack_bf16x2(grp[0], grp[1]), pack_bf16x2(grp[2], grp[3]));
                } else {
#pragma unroll
                  for (int j = 0; j < 4; ++j) PhQ[FULL ? tok : 0][F0 + f - 3 + j] = grp[j];
                }
              }
            } else {
              if constexpr (BF) {
                PhK[F0 + f][tok] = __builtin_bit_cast(uint16_t, f32_to_bf16(val));
              } else {
                PhK[tok][F0 + f] = val;
              }
            }
          });
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

    if constexpr (FULL) {
      // ---- phase 3: masked polynomial block P ------------------------------
      for (int tt = w; tt < NTT; tt += 4) {
        const int tok = 16 * tt + li;
        bf16x4 bq = {};
        if constexpr (BF) bq = __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(&Xqb[tok][4 * g]));
        const int ktmax = min(tt | 1, NTT - 1);
        for (int kt = 0; kt <= ktmax; ++kt) {
          float p[4] = {0.f, 0.f, 0.f, 0.f};
          if (kt <= tt) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
            if constexpr (BF) {
              const bf16x4 ak = __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(&Xkb[16 * kt + li][4 * g]));
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
            *reinterpret_cast<uint2*>(&P[tok][16 * kt + 4 * g]) =
                make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) P[tok][16 * kt + 4 * g + r] = p[r];
          }
        }
      }
    }
    __syncthreads();

    if constexpr (FULL) {
      // ---- phase 4: Y = phi_hat(Q) S + P V and the normaliser --------------
      if constexpr (BF) {
        bf16x8 bs[NFT / 2];
#pragma unroll
        for (int kb = 0; kb < NFT / 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            bs[kb][r] = f32_to_bf16(Sacc[2 * kb][r]);
            bs[kb][4 + r] = f32_to_bf16(Sacc[2 * kb + 1][r]);
          }
        const uint32_t one2 = li == 0 ? 0x3F803F80u : 0u;  // bfloat16 1.0 pair in column 0
        const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(one2, one2, one2, one2));
        const uint16_t* tsrc = li == 0 ? Thb : Tlb;
#pragma unroll
        for (int mt = 0; mt < NTT; ++mt) {
          const int tok = 16 * mt + li;
          f32x4 y = {0.f, 0.f, 0.f, 0.f};
          f32x4 yd = {0.f, 0.f, 0.f, 0.f};
          const bool mine = (mt & 3) == w;  // this wave produces the normaliser of token tile mt
#pragma unroll
          for (int kb = 0; kb < NFT / 2; ++kb) {
            const uint2 lo = *reinterpret_cast<const uint2*>(&PhQ[tok][32 * kb + 4 * g]);
            const uint2 hi = *reinterpret_cast<const uint2*>(&PhQ[tok][32 * kb + 16 + 4 * g]);
            const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
            y = mfma_bf16_k32(a, bs[kb], y);
            if (mine) {
              // T as B column 0 (high part) and column 1 (low part), same k-slot order
              uint2 t0 = *reinterpret_cast<const uint2*>(&tsrc[32 * kb + 4 * g]);
              uint2 t1 = *reinterpret_cast<const uint2*>(&tsrc[32 * kb + 16 + 4 * g]);
              if (li >= 2) t0 = t1 = make_uint2(0, 0);
              yd = mfma_bf16_k32(a, __builtin_bit_cast(bf16x8, make_uint4(t0.x, t0.y, t1.x, t1.y)), yd);
            }
          }
          const int nkb = (16 * mt + 15) / 32 + 1;
          for (int kb = 0; kb < nkb; ++kb) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&P[tok][32 * kb + 8 * g]));
            const uint4 b4 = *reinterpret_cast<const uint4*>(&Vl[col][32 * kb + 8 * g]);
            y = mfma_bf16_k32(a, __builtin_bit_cast(bf16x8, b4), y);
            if (mine) yd = mfma_bf16_k32(a, ones, yd);  // row sums of P into column 0
          }
          Y[mt] = y;
          if (mine) {
            // lanes li = 0 / 1 hold column 0 / 1 for tokens 16mt + 4g + r
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float dn = yd[r] + __shfl_down(yd[r], 1);
              if (li == 0) invden[16 * mt + 4 * g + r] = 1.0f / dn;
            }
          }
        }
      } else {
        const float one = li == 0 ? 1.0f : 0.0f;
#pragma unroll
        for (int mt = 0; mt < NTT; ++mt) {
          const int tok = 16 * mt + li;
          f32x4 y = {0.f, 0.f, 0.f, 0.f};
          f32x4 yd = {0.f, 0.f, 0.f, 0.f};
          const bool mine = (mt & 3) == w;
#pragma unroll
          for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float a = PhQ[tok][16 * ft + 4 * g + r];
              y = mfma_f32_k4(a, Sacc[ft][r], y);
              if (mine) yd = mfma_f32_k4(a, li == 0 ? Ts[16 * ft + 4 * g + r] : 0.0f, yd);
            }
          const int nst = (16 * mt + 16) / 4;
          for (int st = 0; st < nst; ++st) {
            const float a = P[tok][4 * st + g];
            y = mfma_f32_k4(a, Vl[4 * st + g][col], y);
            if (mine) yd = mfma_f32_k4(a, one, yd);
          }
          Y[mt] = y;
          if (mine && li == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) invden[16 * mt + 4 * g + r] = 1.0f / yd[r];
          }
        }
      }
      prev_t0 = t0;
      prev_nv = nv;
    }

    // ---- phase 5: S += phi(K)^T V and T += phi(K)^T 1 ----------------------
    if constexpr (BF) {
      const uint32_t one2 = li == 0 ? 0x3F803F80u : 0u;
      const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(one2, one2, one2, one2));
#pragma unroll
      for (int kb = 0; kb < C / 32; ++kb) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&Vl[col][32 * kb + 8 * g]));
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
          const bf16x8 a =
              __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&PhK[16 * ft + li][32 * kb + 8 * g]));
          Sacc[ft] = mfma_bf16_k32(a, b, Sacc[ft]);
          if ((ft & 3) == w) Tacc[ft >> 2] = mfma_bf16_k32(a, ones, Tacc[ft >> 2]);
        }
      }
    } else {
      const float one = li == 0 ? 1.0f : 0.0f;
      for (int st = 0; st < C / 4; ++st) {
        const float b = Vl[4 * st + g][col];
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
          const float a = PhK[4 * st + g][16 * ft + li];
          Sacc[ft] = mfma_f32_k4(a, b, Sacc[ft]);
          if ((ft & 3) == w) Tacc[ft >> 2] = mfma_f32_k4(a, one, Tacc[ft >> 2]);
        }
      }
    }
    __syncthreads();
  }
  epilogue();

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
    if (li == 0) {
#pragma unroll
      for (int j = 0; j < Sh::NTW; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * (w + 4 * j) + 4 * g + r;
          if (w + 4 * j < NFT && row < D) dst_T[slot * D + row] = Tacc[j][r];
        }
    }
  }
}

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
  p.nchunks = (N + chunk - 1) / chunk;
  // Aim for at least 512 workgroups in the chunk kernel (two per CU on a
  // 256-CU part) when the heads alone do not provide them; 128-token chunks
  // fill an LDS on their own, so for them aim at one workgroup per CU.  In
  // the feature-blocked kernel (d = 16 with n >= 4, and d = 32, 64) every
  // segment is split into feature blocks, one workgroup each.
  const bool fbk = prefill_uses_fb(d, n);
  const int blocks = fbk ? prefill_fb_blocks(d, n) : 1;
  const int target = chunk >= 128 ? 256 : 512;
  // feature-blocked: at most one round of workgroups (a second, partial round
  // would cost as much as the first)
  int nseg = fbk ? target / (BH * blocks) : (target + BH * blocks - 1) / (BH * blocks);
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
  if (fbk) {
    const size_t out = prefill_fb_output_floats(BH, N, d, n);
    if (out > 0) p.workspace_floats = (p.workspace_floats + 3) / 4 * 4 + out;  // 16-byte aligned partial outputs
  }
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
    if (hipError_t e = launch_segment_scan(st_S, st_T, W_S, W_T, D, pl.nseg, a.BH, a.stream)) return e;
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
  if (a.d == kD && a.n == 3 && a.in_bf16 && (a.chunk == 64 || a.chunk == 128)) return launch_prefill_n3_bf16(a);
  if (prefill_uses_fb(a.d, a.n)) return launch_prefill_fb(a);
  switch (a.n) {
    case 1: return launch_prefill_n<1>(a);
    case 2: return launch_prefill_n<2>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace taylor
