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
//   * exp2 of (score * log2(e) / a - m) on the vector ALU.
//   * O^T += V^T P^T on the matrix cores: the lane's weights are already in
//     the B-operand layout (query li, keys of its lane group), and the output
//     O^T has the query on the lane as well, so the rescale by exp2(m_old -
//     m_new) is one multiply per accumulator.  V^T comes from LDS: every wave
//     loads 16 keys of V as natural 16-byte row pieces and transposes them on
//     the matrix cores (a product with one-hot operands, exact for bfloat16),
//     so the LDS stores are 8-byte rows; double-buffered, one barrier per key
//     block.
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
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[4] = {zero, zero, zero, zero};  // O^T: lane (li, g) holds columns 16 ct + 4g + r of query li
  float m = -__builtin_inff(), lsum = 0.0f;

  for (int kb = 0; kb <= qb; ++kb) {
    const int k0 = kb * kKB, buf = kb & 1;
    // V^T of this wave's 16 keys: A = rows of V (key li, columns 8g..8g+7 and
    // 32+8g..), times the one-hot operands -> lane (column li, g) holds keys
    // 4g..4g+3 of the tile
    {
      const int key = k0 + 16 * w + li;
      const size_t r = base + min(key, N - 1);
      const uint4 z4 = make_uint4(0, 0, 0, 0);
      const uint4 ra = *reinterpret_cast<const uint4*>(v + r * kDV + 8 * g);
      const uint4 rb = *reinterpret_cast<const uint4*>(v + r * kDV + 32 + 8 * g);
      const bf16x8 va = __builtin_bit_cast(bf16x8, key < N ? ra : z4);
      const bf16x8 vb = __builtin_bit_cast(bf16x8, key < N ? rb : z4);
      const f32x4 d[4] = {mfma_bf16_k32(va, sel0, zero), mfma_bf16_k32(va, sel1, zero),
                          mfma_bf16_k32(vb, sel0, zero), mfma_bf16_k32(vb, sel1, zero)};
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        *reinterpret_cast<uint2*>(&VT[buf][16 * ct + li][16 * w + 4 * g]) =
            make_uint2(pack2(d[ct][0], d[ct][1]), pack2(d[ct][2], d[ct][3]));
    }
    // scores: S^T = K Q^T per 16-key tile; lane (li, g) gets keys 16 kt + 4g + r of query li
    f32x4 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int key = min(k0 + 16 * kt + li, N - 1);
      const bf16x4 ak = __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(k + (base + key) * kD + 4 * g));
      s[kt] = mfma_bf16_k16(ak, bq, zero);
    }
    __syncthreads();  // V^T of the block is in LDS

    // log2-domain scores; keys after the query (and past N) get -inf.  Only
    // the diagonal block can hold either.
    float x[4][4];
    const bool diag = kb == qb;  // uniform
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 16 * kt + 4 * g + r;
        x[kt][r] = (diag && key > qi) ? -__builtin_inff() : s[kt][r] * scale;
      }
    const float m_new = fmaxf(m, block_max(x));  // finite: key k0 <= qi in every block
    const float alpha = exp2f(m - m_new);        // 0 on the first block (m = -inf)
    uint32_t pw[4][2];
    float psum = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const uint32_t u = pack2(exp2f(x[kt][r] - m_new), exp2f(x[kt][r + 1] - m_new));
        pw[kt][r / 2] = u;
        psum += lo_f(u) + hi_f(u);  // the rounded weights, as used in the product
      }
    }
    lsum = lsum * alpha + psum;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[ct] *= alpha;
    // O^T += V^T P^T over the two 32-key halves: k-slots 8g..8g+3 are keys
    // 32h + 4g + r, k-slots 8g+4..8g+7 keys 32h + 16 + 4g + r, on both sides
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16x8 bp = __builtin_bit_cast(bf16x8, make_uint4(pw[2 * h][0], pw[2 * h][1], pw[2 * h + 1][0],
                                                               pw[2 * h + 1][1]));
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const uint2 a0 = *reinterpret_cast<const uint2*>(&VT[buf][16 * ct + li][32 * h + 4 * g]);
        const uint2 a1 = *reinterpret_cast<const uint2*>(&VT[buf][16 * ct + li][32 * h + 16 + 4 * g]);
        acc[ct] = mfma_bf16_k32(__builtin_bit_cast(bf16x8, make_uint4(a0.x, a0.y, a1.x, a1.y)), bp, acc[ct]);
      }
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
    const float alpha = exp2f(m - m_new);
    float p[4][4], psum = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[kt][r] = exp2f(x[kt][r] - m_new);
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
