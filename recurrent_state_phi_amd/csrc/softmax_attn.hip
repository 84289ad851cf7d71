// Exact causal softmax attention on gfx950: Eq. (1) of "A Taylor-Series Route
// to Linear-Time Transformers with a Fixed Number of Recurrent States"
// (arXiv 2610.20637), o_t = sum_{i<=t} exp(q_t.k_i / a) v_i / sum_{i<=t} exp(q_t.k_i / a),
// the method the paper measures the Taylor states against (prefill in
// section 5.5, decode against a growing key-value cache in section 5.6).
//
// Prefill: one workgroup of 4 waves per (head, 64-query block); wave w owns
// queries 16w..16w+15 of the block and walks the key blocks 0..qb in order,
// keeping a running maximum m and a running normaliser l per query (the
// rescaling form of the softmax: exp(x - m) with m the running maximum,
// which cancels in the ratio and keeps every exponent <= 0).
//   * Scores S^T = K Q^T per 16-key tile on the matrix cores: lane (li, g)
//     ends up with query li and keys 16 kt + 4g + r -- for one query, 16 of
//     the block's 64 keys per lane, the other 48 in the lanes 16 and 32 apart.
//   * exp2 of (score * log2(e) / a - m) on the vector ALU, straight on the
//     hardware exponential.  m is moved (and the accumulators rescaled) only
//     when a row's block maximum exceeds it by more than 8 in log2 units, so
//     most blocks skip the cross-lane maximum and the rescale; the weights
//     stay <= 2^8, and any m shared by the lanes of a query cancels exactly.
//   * O^T += V^T P^T on the matrix cores: the lane's weights are already in
//     the B-operand layout (query li, keys of its lane group), and the output
//     O^T has the query on the lane as well, so the rescale by exp2(m_old -
//     m_new) is one multiply per accumulator.  V^T comes from LDS: every wave
//     loads 32 keys x 32 columns of V as natural 16-byte row pieces and
//     transposes them on the matrix cores (a product with one-hot operands,
//     exact for bfloat16), storing them in the k-slot order of the products,
//     so LDS is written and read in 16-byte row pieces (row stride 144 bytes:
//     16 lanes of a 16-byte access cover all 64 banks once); double-buffered,
//     one barrier per key block.
//   bfloat16 inputs: bfloat16 operands, float32 accumulation, the weights
//   rounded to bfloat16 for the product and the normaliser summed from the
//   same rounded weights (so the output is an exact weighted mean of the
//   rows of V with those weights).  float32 inputs: float32 operands
//   (16x16x4 float32 products) and float32 weights throughout.
//
// Decode: per step, the new key and value go into the cache at position pos
// and the query attends over positions 0..pos.  The keys are split into
// ranges of 2048 per workgroup (split-K); a thread handles keys
// slot, slot + 64, ... of its range (64 slots, 4 threads per key, each
// holding 4 of the 16 key dimensions and 16 of the 64 value columns), keeps
// its own (m, l, o) and the partial results are merged -- across lanes,
// across waves, then across ranges in a second small kernel -- by the same
// rescaling rule.  The step reads the whole cache once: bound by HBM.
#include <type_traits>

#include "taylor_device.h"
#include "taylor_launch.h"

namespace taylor {
namespace sm {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kQB = 64;    // queries per workgroup
constexpr int kKB = 64;    // keys per block
constexpr int kVS = 72;    // row stride (bf16) of V^T in LDS
constexpr int kVF = 68;    // row stride (float) of V in LDS, float32 path
constexpr int kSplit = 2048;  // keys per decode workgroup
constexpr int kPart = 68;     // floats per decode partial: m, l, 2 pad, 64 values
constexpr int kBufWord3 = 0x00020000;  // buffer descriptor word 3 (gfx9: 32-bit data, raw)

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const bf16x2 p = {f32_to_bf16(lo), f32_to_bf16(hi)};
  return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ float lo_f(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_f(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

template <typename TOUT>
__device__ __forceinline__ void store4(TOUT* p, f32x4 x) {
  if constexpr (std::is_same_v<TOUT, float>) {
    *reinterpret_cast<f32x4*>(p) = x;
  } else {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack2(x[0], x[1]), pack2(x[2], x[3]));
  }
}

// Running maximum of the 64 scores of one query in a key block: the lane's 16,
// then across the lanes 16 and 32 apart (same query, other keys).
__device__ __forceinline__ float block_max(const float (&x)[4][4]) {
  float mx = x[0][0];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, x[kt][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  return mx;
}

// ---- prefill, bfloat16 inputs ------------------------------------------------
// exp2 on the hardware unit directly: every argument here is <= 0, and results
// below the smallest normal float are weights too small to matter (they flush
// to zero), so the range handling of exp2f is not needed.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum over the four lane groups (lanes li, li + 16, li + 32, li + 48) on the
// vector ALU: the gfx950 lane swaps exchange rows 0 <-> 1 and 2 <-> 3 of 16
// lanes, then the two halves of 32 lanes.
__device__ __forceinline__ float group_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <typename TOUT>
__global__ __launch_bounds__(256) void prefill_bf16_kernel(const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v, TOUT* __restrict__ o,
                                                           int BH, int N, float scale) {
  __shared__ __align__(16) uint16_t VT[2][kDV][kVS];
  const int nqb = (N + kQB - 1) / kQB;
  // every head's last query block first (the longest rows start earliest);
  // blockIdx % 8 picks the XCD, so the blocks of one head share an L2 when
  // BH is a multiple of 8
  const int bh = blockIdx.x % BH;
  const int qb = nqb - 1 - (int)(blockIdx.x / BH);
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t base = (size_t)bh * N;
  const int qi = qb * kQB + 16 * w + li;  // this lane's query
  const bf16x4 bq = __builtin_bit_cast(
      bf16x4, *reinterpret_cast<const uint2*>(q + (base + min(qi, N - 1)) * kD + 4 * g));

  bf16x8 sel0, sel1;  // one-hot operands: k-slots 0..15 / 16..31 to columns
  {
    uint32_t w0[4], w1[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k0 = 8 * g + 2 * e;
      w0[e] = (k0 == li ? 0x3F80u : 0u) | (k0 + 1 == li ? 0x3F800000u : 0u);
      w1[e] = (k0 == li + 16 ? 0x3F80u : 0u) | (k0 + 1 == li + 16 ? 0x3F800000u : 0u);
    }
    sel0 = __builtin_bit_cast(bf16x8, make_uint4(w0[0], w0[1], w0[2], w0[3]));
    sel1 = __builtin_bit_cast(bf16x8, make_uint4(w1[0], w1[1], w1[2], w1[3]));
  }
  // A operand with ones in row 0: ones . P^T puts the row sums of the rounded
  // weights in row 0 of a tile (lanes 0..15)
  const uint32_t one2 = li == 0 ? 0x3F803F80u : 0u;
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(one2, one2, one2, one2));
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[4] = {zero, zero, zero, zero};  // O^T: lane (li, g) holds columns 16 ct + 4g + r of query li
  f32x4 lacc = zero;                        // row 0: the normaliser of query li
  float m = -__builtin_inff();              // running maximum of the raw scores (see block())
  const float margin = 8.0f / scale;        // 2^8 in weight, in raw score units

  // loads of one key block: wave w stages keys 32h..32h+31 (h = w / 2) of
  // the block for value columns 32c..32c+31 (c = w % 2): lane (li, g) takes
  // columns 32c + 8g..8g+7 of keys 32h + li and 32h + 16 + li; and the four
  // 16-key tiles of K (dimensions 4g..4g+3).  Buffer loads over this head's
  // rows: the key block's offset is a scalar, the lane's offset a constant,
  // and rows past N read as zero (the resource's byte limit).
  const int vh = w >> 1, vc = w & 1;
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(v + base * kDV), 0, N * kDV * 2, kBufWord3);
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(k + base * kD), 0, N * kD * 2, kBufWord3);
  const int vo0 = (32 * vh + li) * kDV * 2 + (32 * vc + 8 * g) * 2, vo1 = vo0 + 16 * kDV * 2;
  const int ko = li * kD * 2 + 8 * g;
  uint4 pv[2];
  uint2 pk[4];
  auto issue = [&](int kb) {
    const int k0 = kb * kKB;
    pv[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, vo0, k0 * kDV * 2, 0));
    pv[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, vo1, k0 * kDV * 2, 0));
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      pk[kt] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rk, ko + 16 * kt * kD * 2,
                                                                              k0 * kD * 2, 0));
  };

  auto block = [&](int kb, auto diag_c) {
    constexpr bool DIAG = decltype(diag_c)::value;
    const int k0 = kb * kKB, buf = kb & 1;
    // V^T of this wave's 32 keys x 32 columns into LDS, in the k-slot order
    // of the P.V products (row = value column, slot 8g + r = key 4g + r and
    // slot 8g + 4 + r = key 16 + 4g + r of the 32-key half): the one-hot
    // products give lane (column li, g) keys 4g..4g+3 of each 16-key tile, so
    // its 8 slots are one 16-byte row piece.  And the scores S^T = K Q^T.
    f32x4 s[4];
    {
      const bf16x8 v0 = __builtin_bit_cast(bf16x8, pv[0]), v1 = __builtin_bit_cast(bf16x8, pv[1]);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) s[kt] = mfma_bf16_k16(__builtin_bit_cast(bf16x4, pk[kt]), bq, zero);
      const f32x4 d00 = mfma_bf16_k32(v0, sel0, zero), d01 = mfma_bf16_k32(v0, sel1, zero);
      const f32x4 d10 = mfma_bf16_k32(v1, sel0, zero), d11 = mfma_bf16_k32(v1, sel1, zero);
      if (kb < qb) issue(kb + 1);  // uniform: the next block's loads fly during this block
      *reinterpret_cast<uint4*>(&VT[buf][32 * vc + li][32 * vh + 8 * g]) =
          make_uint4(pack2(d00[0], d00[1]), pack2(d00[2], d00[3]), pack2(d10[0], d10[1]), pack2(d10[2], d10[3]));
      *reinterpret_cast<uint4*>(&VT[buf][32 * vc + 16 + li][32 * vh + 8 * g]) =
          make_uint4(pack2(d01[0], d01[1]), pack2(d01[2], d01[3]), pack2(d11[0], d11[1]), pack2(d11[2], d11[3]));
    }
    // keys after the query (and past N) only occur in the diagonal block
    if constexpr (DIAG) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s[kt][r] = k0 + 16 * kt + 4 * g + r > qi ? -__builtin_inff() : s[kt][r];
    }
    float mx = s[0][0];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kt][r]);
    // The running maximum m moves only when some row's block maximum exceeds
    // it by more than `margin` (8 in log2 units): any m common to the four
    // lane groups of a query leaves the ratio unchanged, and with this rule
    // every weight stays <= 2^8.  On the first block m = -inf, so it is set.
    if (__any(mx > m + margin)) {  // uniform
      mx = group_max(mx);
      const float m_new = fmaxf(m, mx);  // finite: key k0 <= qi in every block
      const float alpha = fast_exp2((m - m_new) * scale);  // 0 while m = -inf
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[ct] *= alpha;
      lacc *= alpha;
      m = m_new;
    }
    const float off = m * scale;
    uint32_t pw[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; r += 2)
        pw[kt][r / 2] = pack2(fast_exp2(fmaf(s[kt][r], scale, -off)), fast_exp2(fmaf(s[kt][r + 1], scale, -off)));
    __syncthreads();  // V^T of the block is in LDS
    // O^T += V^T P^T over the two 32-key halves: k-slots 8g..8g+3 are keys
    // 32h + 4g + r, k-slots 8g+4..8g+7 keys 32h + 16 + 4g + r, on both sides
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16x8 bp = __builtin_bit_cast(bf16x8, make_uint4(pw[2 * h][0], pw[2 * h][1], pw[2 * h + 1][0],
                                                               pw[2 * h + 1][1]));
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const uint4 a = *reinterpret_cast<const uint4*>(&VT[buf][16 * ct + li][32 * h + 8 * g]);
        acc[ct] = mfma_bf16_k32(__builtin_bit_cast(bf16x8, a), bp, acc[ct]);
      }
      lacc = mfma_bf16_k32(ones, bp, lacc);
    }
  };

  issue(0);
  for (int kb = 0; kb < qb; ++kb) block(kb, std::false_type{});
  block(qb, std::true_type{});

  const float l = __shfl(lacc[0], li);  // row 0 of the tile sits in lanes 0..15
  if (qi < N) {
    const float inv = 1.0f / l;
    TOUT* orow = o + (base + qi) * kDV + 4 * g;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) store4<TOUT>(orow + 16 * ct, acc[ct] * inv);
  }
}

// ---- prefill, float32 inputs -------------------------------------------------
template <typename TOUT>
__global__ __launch_bounds__(256) void prefill_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                          const float* __restrict__ v, TOUT* __restrict__ o, int BH,
                                                          int N, float scale) {
  __shared__ __align__(16) float Vs[2][kKB][kVF];
  const int nqb = (N + kQB - 1) / kQB;
  const int bh = blockIdx.x % BH;
  const int qb = nqb - 1 - (int)(blockIdx.x / BH);
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t base = (size_t)bh * N;
  const int qi = qb * kQB + 16 * w + li;
  // B operand of the four 16x16x4 products: q[query li][4g + i] for product i
  const f32x4 qv = *reinterpret_cast<const f32x4*>(q + (base + min(qi, N - 1)) * kD + 4 * g);
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[4] = {zero, zero, zero, zero};
  float m = -__builtin_inff(), lsum = 0.0f;

  for (int kb = 0; kb <= qb; ++kb) {
    const int k0 = kb * kKB, buf = kb & 1;
    {  // V rows of this wave's 16 keys into LDS (row-major, 16-byte pieces)
      const int key = k0 + 16 * w + li;
      const float* src = v + (base + min(key, N - 1)) * kDV + 16 * g;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(src + 4 * e);
        *reinterpret_cast<f32x4*>(&Vs[buf][16 * w + li][16 * g + 4 * e]) = key < N ? x : zero;
      }
    }
    f32x4 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int key = min(k0 + 16 * kt + li, N - 1);
      const f32x4 kv = *reinterpret_cast<const f32x4*>(k + (base + key) * kD + 4 * g);
      f32x4 t = zero;
#pragma unroll
      for (int i = 0; i < 4; ++i) t = mfma_f32_k4(kv[i], qv[i], t);
      s[kt] = t;
    }
    __syncthreads();

    float x[4][4];
    const bool diag = kb == qb;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 16 * kt + 4 * g + r;
        x[kt][r] = (diag && key > qi) ? -__builtin_inff() : s[kt][r] * scale;
      }
    const float m_new = fmaxf(m, block_max(x));
    const float alpha = fast_exp2(m - m_new);
    float p[4][4], psum = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[kt][r] = fast_exp2(x[kt][r] - m_new);
        psum += p[kt][r];
      }
    lsum = lsum * alpha + psum;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[ct] *= alpha;
    // O^T += V^T P^T, one product per (kt, r): k-slot g is key 16 kt + 4g + r
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = 16 * kt + 4 * g + r;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[ct] = mfma_f32_k4(Vs[buf][key][16 * ct + li], p[kt][r], acc[ct]);
      }
    m = m_new;
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (qi < N) {
    const float inv = 1.0f / lsum;
    TOUT* orow = o + (base + qi) * kDV + 4 * g;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) store4<TOUT>(orow + 16 * ct, acc[ct] * inv);
  }
}

// ---- decode -----------------------------------------------------------------
template <typename T> struct Vec;
template <> struct Vec<uint16_t> {  // 4 keys dims / 16 value columns of bfloat16
  static __device__ __forceinline__ void load_k(const uint16_t* p, float (&x)[4]) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    x[0] = lo_f(u.x); x[1] = hi_f(u.x); x[2] = lo_f(u.y); x[3] = hi_f(u.y);
  }
  static __device__ __forceinline__ void load_v(const uint16_t* p, float (&x)[16]) {
    const uint4 a = *reinterpret_cast<const uint4*>(p), b = *reinterpret_cast<const uint4*>(p + 8);
    const uint32_t u[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = lo_f(u[i]);
      x[2 * i + 1] = hi_f(u[i]);
    }
  }
  static __device__ __forceinline__ void copy_k(uint16_t* d, const uint16_t* s) {
    *reinterpret_cast<uint2*>(d) = *reinterpret_cast<const uint2*>(s);
  }
  static __device__ __forceinline__ void copy_v(uint16_t* d, const uint16_t* s) {
    reinterpret_cast<uint4*>(d)[0] = reinterpret_cast<const uint4*>(s)[0];
    reinterpret_cast<uint4*>(d)[1] = reinterpret_cast<const uint4*>(s)[1];
  }
};
template <> struct Vec<float> {
  static __device__ __forceinline__ void load_k(const float* p, float (&x)[4]) {
    const f32x4 u = *reinterpret_cast<const f32x4*>(p);
    x[0] = u[0]; x[1] = u[1]; x[2] = u[2]; x[3] = u[3];
  }
  static __device__ __forceinline__ void load_v(const float* p, float (&x)[16]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 u = reinterpret_cast<const f32x4*>(p)[i];
      x[4 * i] = u[0]; x[4 * i + 1] = u[1]; x[4 * i + 2] = u[2]; x[4 * i + 3] = u[3];
    }
  }
  static __device__ __forceinline__ void copy_k(float* d, const float* s) {
    *reinterpret_cast<f32x4*>(d) = *reinterpret_cast<const f32x4*>(s);
  }
  static __device__ __forceinline__ void copy_v(float* d, const float* s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) reinterpret_cast<f32x4*>(d)[i] = reinterpret_cast<const f32x4*>(s)[i];
  }
};

// (m, l, o) <- merge of (m, l, o) and (m2, l2, o2) by the rescaling rule; an
// empty side has m = -inf and l = o = 0.
template <int NV>
__device__ __forceinline__ void merge(float& m, float& l, float (&o)[NV], float m2, float l2, const float (&o2)[NV]) {
  const float M = fmaxf(m, m2);
  const bool empty = M == -__builtin_inff();
  const float c1 = empty ? 0.0f : exp2f(m - M), c2 = empty ? 0.0f : exp2f(m2 - M);
  l = l * c1 + l2 * c2;
#pragma unroll
  for (int i = 0; i < NV; ++i) o[i] = o[i] * c1 + o2[i] * c2;
  m = M;
}

template <typename TIN>
__global__ __launch_bounds__(256) void decode_partial_kernel(const TIN* __restrict__ q, const TIN* __restrict__ kn,
                                                             const TIN* __restrict__ vn, TIN* __restrict__ kc,
                                                             TIN* __restrict__ vc, float* __restrict__ part, int cap,
                                                             int pos, int nsplit, float scale) {
  __shared__ float red[4][4][2 + 16];  // [wave][quad][m, l, 16 values]
  const int bh = blockIdx.x / nsplit, sp = blockIdx.x % nsplit;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, quad = tid & 3, slot = tid >> 2;
  const int kbeg = sp * kSplit;
  const int kend = min(pos, kbeg + kSplit);  // cached keys of this range; key pos comes from the inputs
  const size_t hc = (size_t)bh * cap;
  float qv[4];
  Vec<TIN>::load_k(q + (size_t)bh * kD + 4 * quad, qv);
#pragma unroll
  for (int i = 0; i < 4; ++i) qv[i] *= scale;  // scores in log2 units
  float m = -__builtin_inff(), l = 0.0f, acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;

  // 4 keys per thread per round, loads of all four in flight together
  for (int key0 = kbeg + slot; key0 < kend; key0 += 256) {
    float s[4], vv[4][16];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t r = hc + min(key0 + 64 * u, kend - 1);
      float kk[4];
      Vec<TIN>::load_k(kc + r * kD + 4 * quad, kk);
      Vec<TIN>::load_v(vc + r * kDV + 16 * quad, vv[u]);
      s[u] = qv[0] * kk[0] + qv[1] * kk[1] + qv[2] * kk[2] + qv[3] * kk[3];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      s[u] += __shfl_xor(s[u], 1);
      s[u] += __shfl_xor(s[u], 2);
      s[u] = key0 + 64 * u < kend ? s[u] : -__builtin_inff();
    }
    const float m_new = fmaxf(fmaxf(m, fmaxf(s[0], s[1])), fmaxf(s[2], s[3]));  // finite: s[0] is a key
    const float c = exp2f(m - m_new);
    float p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) p[u] = exp2f(s[u] - m_new);
    l = l * c + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
    for (int i = 0; i < 16; ++i)
      acc[i] = acc[i] * c + ((p[0] * vv[0][i] + p[1] * vv[1][i]) + (p[2] * vv[2][i] + p[3] * vv[3][i]));
    m = m_new;
  }
  // the new token (the last range holds position pos): the four threads of
  // slot 0 read it from the inputs, write it into the cache and take it in
  if (sp == nsplit - 1 && slot == 0) {
    float kk[4], vv[16];
    Vec<TIN>::load_k(kn + (size_t)bh * kD + 4 * quad, kk);
    Vec<TIN>::load_v(vn + (size_t)bh * kDV + 16 * quad, vv);
    Vec<TIN>::copy_k(kc + (hc + pos) * kD + 4 * quad, kn + (size_t)bh * kD + 4 * quad);
    Vec<TIN>::copy_v(vc + (hc + pos) * kDV + 16 * quad, vn + (size_t)bh * kDV + 16 * quad);
    float s = qv[0] * kk[0] + qv[1] * kk[1] + qv[2] * kk[2] + qv[3] * kk[3];
    s += __shfl_xor(s, 1);  // lanes 0..3 of wave 0 are all active here
    s += __shfl_xor(s, 2);
    float one[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) one[i] = vv[i];
    merge<16>(m, l, acc, s, 1.0f, one);
  }
  // merge the 16 slots of the wave (lanes 4, 8, 16, 32 apart hold the same columns)
#pragma unroll
  for (int off = 4; off <= 32; off <<= 1) {
    float o2[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) o2[i] = __shfl_xor(acc[i], off);
    const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
    merge<16>(m, l, acc, m2, l2, o2);
  }
  if (lane < 4) {
    red[w][quad][0] = m;
    red[w][quad][1] = l;
#pragma unroll
    for (int i = 0; i < 16; ++i) red[w][quad][2 + i] = acc[i];
  }
  __syncthreads();
  if (tid < kDV) {  // column tid: quad tid / 16, value tid % 16
    const int qd = tid >> 4, i = tid & 15;
    float mm = red[0][qd][0], ll = red[0][qd][1], oo[1] = {red[0][qd][2 + i]};
#pragma unroll
    for (int wv = 1; wv < 4; ++wv) {
      const float o2[1] = {red[wv][qd][2 + i]};
      merge<1>(mm, ll, oo, red[wv][qd][0], red[wv][qd][1], o2);
    }
    float* dst = part + ((size_t)bh * nsplit + sp) * kPart;
    dst[4 + tid] = oo[0];
    if (tid == 0) {
      dst[0] = mm;
      dst[1] = ll;
    }
  }
}

template <typename TOUT>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ part, TOUT* __restrict__ o,
                                                            int nsplit) {
  const int bh = blockIdx.x, c = threadIdx.x;
  const float* p = part + (size_t)bh * nsplit * kPart;
  float m = p[0], l = p[1], acc[1] = {p[4 + c]};
  for (int s = 1; s < nsplit; ++s) {
    const float o2[1] = {p[s * kPart + 4 + c]};
    merge<1>(m, l, acc, p[s * kPart], p[s * kPart + 1], o2);
  }
  Elem<TOUT>::store(o, (size_t)bh * kDV + c, acc[0] / l);
}

template <typename TIN, typename TOUT>
hipError_t launch_prefill_t(const SoftmaxPrefillArgs& a) {
  const int nqb = (a.N + kQB - 1) / kQB;
  const float scale = kLog2e / a.a;
  const dim3 grid((unsigned)(a.BH * nqb)), block(256);
  if constexpr (std::is_same_v<TIN, uint16_t>) {
    hipLaunchKernelGGL((prefill_bf16_kernel<TOUT>), grid, block, 0, a.stream, static_cast<const uint16_t*>(a.q),
                       static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                       static_cast<TOUT*>(a.o), a.BH, a.N, scale);
  } else {
    hipLaunchKernelGGL((prefill_f32_kernel<TOUT>), grid, block, 0, a.stream, static_cast<const float*>(a.q),
                       static_cast<const float*>(a.k), static_cast<const float*>(a.v), static_cast<TOUT*>(a.o),
                       a.BH, a.N, scale);
  }
  return hipGetLastError();
}

template <typename TIN, typename TOUT>
hipError_t launch_decode_t(const SoftmaxDecodeArgs& a) {
  const int nsplit = softmax_decode_splits(a.pos + 1);
  const float scale = kLog2e / a.a;
  hipLaunchKernelGGL((decode_partial_kernel<TIN>), dim3((unsigned)(a.BH * nsplit)), dim3(256), 0, a.stream,
                     static_cast<const TIN*>(a.q), static_cast<const TIN*>(a.k), static_cast<const TIN*>(a.v),
                     static_cast<TIN*>(a.k_cache), static_cast<TIN*>(a.v_cache), a.workspace, a.cap, a.pos, nsplit,
                     scale);
  hipLaunchKernelGGL((decode_combine_kernel<TOUT>), dim3((unsigned)a.BH), dim3(64), 0, a.stream, a.workspace,
                     static_cast<TOUT*>(a.o), nsplit);
  return hipGetLastError();
}

}  // namespace sm

int softmax_decode_splits(int len) { return (len + sm::kSplit - 1) / sm::kSplit; }
size_t softmax_decode_workspace_floats(int BH, int cap) {
  return (size_t)BH * softmax_decode_splits(cap) * sm::kPart;
}

hipError_t launch_softmax_prefill(const SoftmaxPrefillArgs& a) {
  if (a.in_bf16) return a.out_bf16 ? sm::launch_prefill_t<uint16_t, uint16_t>(a) : sm::launch_prefill_t<uint16_t, float>(a);
  return a.out_bf16 ? sm::launch_prefill_t<float, uint16_t>(a) : sm::launch_prefill_t<float, float>(a);
}

hipError_t launch_softmax_decode(const SoftmaxDecodeArgs& a) {
  if (a.in_bf16) return a.out_bf16 ? sm::launch_decode_t<uint16_t, uint16_t>(a) : sm::launch_decode_t<uint16_t, float>(a);
  return a.out_bf16 ? sm::launch_decode_t<float, uint16_t>(a) : sm::launch_decode_t<float, float>(a);
}

}  // namespace taylor
