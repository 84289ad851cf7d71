// Device-side building blocks for the gfx950 Taylor-state kernels.
//
// Feature map (section 3.4 of "A Taylor-Series Route to Linear-Time
// Transformers with a Fixed Number of Recurrent States", arXiv 2610.20637):
// for order m the features are the monomials x_{i1} x_{i2} ... x_{im} over
// nondecreasing multi-indices i1 <= ... <= im, in lexicographic order, each
// multiplied by sqrt(m! / prod_i c_i!) where c_i counts how often coordinate i
// occurs.  Orders are stacked m = 0, 1, ..., n-1, giving D = sum_m C(d+m-1, m)
// rows.  With these weights <phi_m(q), phi_m(k)> = (q.k)^m exactly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace taylor {

constexpr int kD = 16;   // head dimension of q and k
constexpr int kDV = 64;  // value dimension

constexpr int order_width(int m) {  // C(kD + m - 1, m)
  long r = 1;
  for (int i = 1; i <= m; ++i) r = r * (kD - 1 + i) / i;
  return (int)r;
}
constexpr int state_width(int n) {
  int s = 0;
  for (int m = 0; m < n; ++m) s += order_width(m);
  return s;
}
constexpr int round_up(int x, int r) { return (x + r - 1) / r * r; }

// sqrt-multinomial weights that occur for m <= 3.
constexpr float kSqrt2 = 1.41421356237309504880f;
constexpr float kSqrt3 = 1.73205080756887729353f;
constexpr float kSqrt6 = 2.44948974278317809820f;

// Row descriptor of the stacked basis: order m, coordinates (unused ones 0)
// and the multiplicity weight.  Used where the row index is a runtime value.
struct FeatureTable {
  uint16_t code[969];  // m | i0 << 2 | i1 << 6 | i2 << 10  (bits 0-1: m, 4 bits per index)
  float weight[969];
};

constexpr FeatureTable make_feature_table() {
  FeatureTable t{};
  int f = 0;
  t.code[f] = 0; t.weight[f] = 1.0f; ++f;                                   // m = 0
  for (int i = 0; i < kD; ++i) { t.code[f] = (uint16_t)(1 | i << 2); t.weight[f] = 1.0f; ++f; }
  for (int i = 0; i < kD; ++i)
    for (int j = i; j < kD; ++j) {
      t.code[f] = (uint16_t)(2 | i << 2 | j << 6);
      t.weight[f] = (i == j) ? 1.0f : kSqrt2;
      ++f;
    }
  for (int i = 0; i < kD; ++i)
    for (int j = i; j < kD; ++j)
      for (int l = j; l < kD; ++l) {
        t.code[f] = (uint16_t)(3 | i << 2 | j << 6 | l << 10);
        const int distinct = 1 + (j != i) + (l != j);
        t.weight[f] = distinct == 3 ? kSqrt6 : distinct == 2 ? kSqrt3 : 1.0f;
        ++f;
      }
  return t;
}

// Value of stacked-basis row f at x (kD floats in LDS), scaled by the factor
// of its order: alpha = {alpha_0, alpha_1, alpha_2, alpha_3} with
// alpha_m = 1/(m! a^m) on the query side and all ones on the key side.
// Same, from a row's code and weight already read from the table.
__device__ inline float feature_value(uint32_t c, float weight, const float* x, float4 alpha) {
  const int m = c & 3;
  const float am = m == 0 ? alpha.x : m == 1 ? alpha.y : m == 2 ? alpha.z : alpha.w;
  float v = weight * am;
  if (m >= 1) v *= x[(c >> 2) & 15];
  if (m >= 2) v *= x[(c >> 6) & 15];
  if (m >= 3) v *= x[(c >> 10) & 15];
  return v;
}

__device__ inline float feature_value(const FeatureTable& tab, int f, const float* x, float4 alpha) {
  return feature_value(tab.code[f], tab.weight[f], x, alpha);
}

// D for head dimension d: sum_{m<n} C(d + m - 1, m).
constexpr int state_width_d(int d, int n) {
  int s = 0;
  for (int m = 0; m < n; ++m) {
    long r = 1;
    for (int i = 1; i <= m; ++i) r = r * (d - 1 + i) / i;
    s += (int)r;
  }
  return s;
}

// Rows of the stacked basis (section 3.4) for head dimension KD and orders up
// to MAXM, for kernels that index rows at run time.  Row order as in the
// caller's layout: m ascending, nondecreasing multi-indices i_1 <= ... <= i_m
// in lexicographic order.  Code of a row: bits 0-2 the order m, then MAXM
// fields of kCB bits holding the coordinates, then the multinomial
// m! / prod_i c_i! (at most 120), whose square root is the row's weight.
//   RowTable<16, 5>: n <= 6 at d = 16 (20,349 rows, 4-bit coordinates)
//   RowTable<32, 2>, RowTable<64, 2>: n <= 3 at d = 32, 64 (561, 2,145 rows)
template <int KD, int MAXM>
struct RowTable {
  static constexpr int kCB = KD <= 16 ? 4 : 6;  // bits per coordinate
  static constexpr int kMultShift = 3 + kCB * MAXM;
  static constexpr int kRows = state_width_d(KD, MAXM + 1);
  static_assert(kMultShift + 7 <= 32, "row code fits 32 bits");
  uint32_t code[kRows];
};

template <int KD, int MAXM>
constexpr RowTable<KD, MAXM> make_row_table() {
  using T = RowTable<KD, MAXM>;
  T t{};
  int f = 0;
  for (int m = 0; m <= MAXM; ++m) {
    int idx[MAXM + 1] = {};
    while (true) {
      uint32_t mult = 1;  // m! / prod_i c_i!, built up one coordinate at a time
      for (int p = 0, run = 0; p < m; ++p) {
        run = (p > 0 && idx[p] == idx[p - 1]) ? run + 1 : 1;
        mult = mult * (p + 1) / run;
      }
      uint32_t c = (uint32_t)m | mult << T::kMultShift;
      for (int p = 0; p < m; ++p) c |= (uint32_t)idx[p] << (3 + T::kCB * p);
      t.code[f++] = c;
      int p = m - 1;  // next nondecreasing multi-index in lexicographic order
      while (p >= 0 && idx[p] == KD - 1) --p;
      if (p < 0) break;
      ++idx[p];
      for (int r = p + 1; r < m; ++r) idx[r] = idx[p];
    }
  }
  return t;
}

// Coordinate p of a row code (meaningful for p < m).
template <int KD, int MAXM>
__device__ inline int row_coord(uint32_t c, int p) {
  using T = RowTable<KD, MAXM>;
  return (int)((c >> (3 + T::kCB * p)) & ((1u << T::kCB) - 1));
}
// The row's sqrt-multinomial weight.
template <int KD, int MAXM>
__device__ inline float row_weight(uint32_t c) {
  return __fsqrt_rn((float)(c >> RowTable<KD, MAXM>::kMultShift));
}
// Value of a row at x (KD floats, e.g. in LDS), times `scale` (alpha_m on the
// query side, 1 on the key side).
template <int KD, int MAXM>
__device__ inline float row_feature_value(uint32_t c, const float* x, float scale) {
  const int m = c & 7;
  float v = scale * row_weight<KD, MAXM>(c);
#pragma unroll
  for (int p = 0; p < MAXM; ++p)
    if (p < m) v *= x[row_coord<KD, MAXM>(c, p)];
  return v;
}

// alpha_m = 1 / (m! a^m) (query side) for the order m of a RowTable
// row, given 1/a.  The six factors are plain values and the choice a chain of
// selects between them (a table in memory indexed per lane would go to
// scratch); in a loop they are computed once.
__device__ inline float alpha_of(float inv_a, uint32_t c) {
  const int m = c & 7;
  const float a1 = inv_a, a2 = a1 * inv_a / 2.0f, a3 = a2 * inv_a / 3.0f;
  const float a4 = a3 * inv_a / 4.0f, a5 = a4 * inv_a / 5.0f;
  float r = 1.0f;
  r = m == 1 ? a1 : r;
  r = m == 2 ? a2 : r;
  r = m == 3 ? a3 : r;
  r = m == 4 ? a4 : r;
  r = m == 5 ? a5 : r;
  return r;
}

// Compile-time enumeration of rows [F0, F1) of the stacked basis for n <= 3,
// calling fn(f, value) with f relative to F0.  Rows >= D give 0 (padding).
// All indices are compile-time constants after unrolling, so x stays in
// registers.  `am` holds the per-order factors {alpha_0, alpha_1, alpha_2}.
template <int NT, int F0, int F1, typename Fn>
__device__ __forceinline__ void for_features(const float (&x)[kD], const float (&am)[3], Fn&& fn) {
  constexpr int D = state_width(NT);
  if constexpr (F0 <= 0 && 0 < F1) fn(0 - F0, am[0]);
  if constexpr (NT >= 2) {
#pragma unroll
    for (int i = 0; i < kD; ++i) {
      const int f = 1 + i;
      if (f >= F0 && f < F1) fn(f - F0, am[1] * x[i]);
    }
  }
  if constexpr (NT >= 3) {
#pragma unroll
    for (int i = 0; i < kD; ++i) {
      const float xi = x[i] * am[2];
      const float xi2 = xi * kSqrt2;
#pragma unroll
      for (int j = i; j < kD; ++j) {
        const int f = 1 + kD + i * kD - (i * (i - 1)) / 2 + (j - i);
        if (f >= F0 && f < F1) fn(f - F0, (j == i ? xi : xi2) * x[j]);
      }
    }
  }
#pragma unroll
  for (int f = (D > F0 ? D : F0); f < F1; ++f) fn(f - F0, 0.0f);
}

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// 16x16 output tiles.  Lane l of a wave holds D[4*(l/16) + r][l % 16], r = 0..3.
// A operand: lane l supplies row (l % 16); B operand: lane l supplies column
// (l % 16); lane group g = l / 16 supplies the k-slots of that group (the same
// k-slot numbering for A and B, which is all the reduction needs).
__device__ __forceinline__ f32x4 mfma_bf16_k32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16_k16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32_k4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }
__device__ __forceinline__ __bf16 f32_to_bf16(float x) { return (__bf16)x; }  // round to nearest even

// Input element loaders: float32 or bfloat16 storage, returned as float.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float x) { p[i] = x; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(uint16_t* p, size_t i, float x) {
    __bf16 b = f32_to_bf16(x);
    p[i] = __builtin_bit_cast(uint16_t, b);
  }
};

// The sequence served by workgroup wg of a segment-parallel prefill launch
// (nseg segments per sequence, nseq sequences, one workgroup per segment).
// The chip hands out workgroups to its 8 XCDs in turn (workgroup wg runs on
// XCD wg mod 8: observed for every workgroup of such a launch), so when nseq
// is a multiple of 8, sequence b goes to workgroups of residue b mod 8 and
// all its segments, which pass their state sums to each other, run on one
// XCD; that took the n = 3 prefill from 59.6 to 56.9 us per call.  Every
// sequence is served by exactly nseg workgroups either way, and nothing else
// depends on where they run.
__device__ __forceinline__ int sequence_of_workgroup(int wg, int nseg, int nseq) {
  return nseq % 8 == 0 ? wg % 8 + 8 * ((wg / 8) / nseg) : wg / nseg;
}

}  // namespace taylor
