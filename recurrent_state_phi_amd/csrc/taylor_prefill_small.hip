// Single-launch prefill for n = 1, 2 at d = 16 (section 3.5 of "A Taylor-Series
// Route to Linear-Time Transformers with a Fixed Number of Recurrent States",
// arXiv 2610.20637): float32 arithmetic, q, k and v read from HBM once.
//
// For n <= 2 the state is small.  With the weight 1 + q.k / a of Eq. (2)
// (n = 2; n = 1 keeps only the 1) it is, in the caller's row order
// (section 3.4, key-side features unscaled):
//     S = [ C = sum v  ;  M = sum k v^T (16 x 64) ],   T = [ count ; K = sum k ].
// With P = tril(p_n(Q K^T / a)) for a chunk of 16 tokens and the state A of
// the tokens before it, the chunk's outputs are (Eq. (5), with Eq. (1)-(2) on
// the diagonal block)
//     Y = C + P V + (Q / a) M,   den = count + rowsum(P) + (Q / a) . K,   o = Y / den,
// and every term is linear in A.  States are additive (section 5.2), so each
// (b, h) sequence is cut into segments of 32 tokens per wave, one workgroup
// each: 8 waves and 256 tokens at n = 2 (one workgroup per CU: its q, k, v
// and state sums fill most of the 160 KB of LDS), 4 waves and 128 tokens at
// n = 1 (two per CU); A before a chunk = caller's state + earlier segments'
// sums + the segment's own tokens before the chunk:
//   1. the workgroup loads its segment's q, k, v into LDS once (zeros past the
//      end of the sequence), and the caller's state into registers;
//   2. wave w sums tokens 32w .. 32w+31 (M on the float32 matrix cores, C, K
//      and the count on the vector ALU) into LDS;
//   3. the segment's sum goes to the workspace at once, with its flag (1);
//   4. while the earlier segments publish, every wave replays its two chunks
//      from the segment's own tokens alone (the earlier waves' sums);
//   5. the prefix over the segments, in groups of G consecutive segments (G =
//      the number of segments up to 32, else about its square root): segment s
//      adds the sums of the earlier members of its group and the totals of the
//      earlier groups, which the last member of each group publishes (flag 2)
//      as soon as it has its own group's part.  One wave polls up to 64 flags
//      in one read (consecutive segments have consecutive flag words); all
//      waves share the image loads, many in flight at a time.  The images and
//      their order are fixed, so results do not depend on timing;
//   6. the prefix's terms (caller's state + earlier segments) are added to
//      each chunk's Y and den, o = Y / den is written;
//   7. the last segment writes caller's state + all segments' sums (the final
//      state) to the caller's state.
// Images and flags carry the segments' sums only; every segment adds the
// caller's state itself.  The final-state write cannot race with those reads:
// a segment raises its flag only after its reads have returned, and the last
// segment writes only after it has seen the flag of every earlier segment of
// its group and of every earlier group's last member, each of which had seen
// its own group's flags.
// Every workgroup serves a fixed sequence (sequence_of_workgroup: all the
// segments of a sequence on one XCD where the dispatch allows) and takes its
// segment from that sequence's ticket counter (the flag word of its last
// segment, which never carries a flag), so a workgroup only waits for segments
// that started before it.  Waits are bounded; one that runs
// out records an error code in the workspace header.  Images cross XCDs
// through buffer accesses with the device-scope cache policy (sc1); a flag goes
// up only after every wave has waited for its image stores and the waves have
// met at a barrier.
#include <hip/hip_ext.h>
#include <type_traits>

#include "taylor_device.h"
#include "taylor_launch.h"

namespace taylor {
namespace small {

// Waves per workgroup: 4 at n = 1 (128-token segments, two workgroups per CU,
// whose phases then overlap), 8 at n = 2, whose 26 times larger images make
// the look-back over twice as many segments cost more than the overlap gains
// (n = 1 / n = 2 on the order sweep: 11.9 / 17.2 us per call with 4 waves,
// 12.3 / 16.2 us with 8).
template <int NT> constexpr int waves_of() { return NT == 1 ? 4 : 8; }
template <int NT> constexpr int threads_of() { return 64 * waves_of<NT>(); }
template <int NT> constexpr int seg_tokens() { return 32 * waves_of<NT>(); }  // 2 chunks of 16 per wave
constexpr int kQS = 20;   // LDS row stride (floats) of q and k
constexpr int kVS = 68;   // LDS row stride (floats) of v
constexpr int kHdr = 64;  // header words: [0] unused, [1] error code, [2] kN3Magic
constexpr int kSC1 = 16;  // buffer cache policy: device scope
constexpr int kBufWord3 = 0x00020000;

// State image (float32): the caller's state layout for one head, S rows of
// 64 then T, padded to whole 16-byte units.  n = 2: C (S row 0), M (S rows
// 1-16), count (T row 0), K (T rows 1-16), 3 floats of padding (1,108 floats);
// n = 1: C, count, 3 floats of padding (68).
template <int NT> struct Img {
  static constexpr int kS = state_width(NT) * kDV;  // floats of S
  static constexpr int kFloats = NT == 2 ? 1108 : 68;
  static constexpr int kVec = kFloats / 4;         // 16-byte units
  static constexpr int kPer = (kVec + threads_of<NT>() - 1) / threads_of<NT>();  // units per thread
  static constexpr int kCnt = kS;                  // T row 0
  static constexpr int kK = kS + 1;                // T rows 1-16 (n = 2)
  static constexpr int kPad = kS + state_width(NT);
};

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const float* p, int floats) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), 0, floats * 4, kBufWord3);
}

__device__ __forceinline__ void raise_flag(int* flag, int value) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(flag, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16-byte unit e of head bh's image, read from or written to the caller's
// state (S of all heads, then T at t_base); padding reads as zero.
template <int NT>
__device__ __forceinline__ f32x4 state_unit_load(const float* state, size_t t_base, int bh, int e) {
  using I = Img<NT>;
  constexpr int D = state_width(NT);
  if (4 * e < I::kS) return *reinterpret_cast<const f32x4*>(state + (size_t)bh * I::kS + 4 * e);
  f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = 4 * e + j - I::kS;
    if (t < D) x[j] = state[t_base + (size_t)bh * D + t];
  }
  return x;
}
template <int NT>
__device__ __forceinline__ void state_unit_store(float* state, size_t t_base, int bh, int e, const f32x4& x) {
  using I = Img<NT>;
  constexpr int D = state_width(NT);
  if (4 * e < I::kS) {
    *reinterpret_cast<f32x4*>(state + (size_t)bh * I::kS + 4 * e) = x;
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = 4 * e + j - I::kS;
    if (t < D) state[t_base + (size_t)bh * D + t] = x[j];
  }
}

// 16 bytes of input as float32 in LDS.
template <typename T> struct Raw;
template <> struct Raw<float> {  // 4 elements
  static constexpr int kPer = 4;
  static __device__ __forceinline__ void put(float* dst, const u32x4& u) {
    *reinterpret_cast<float4*>(dst) = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                                                  __uint_as_float(u.w));
  }
};
template <> struct Raw<uint16_t> {  // 8 elements
  static constexpr int kPer = 8;
  static __device__ __forceinline__ void put(float* dst, const u32x4& u) {
    *reinterpret_cast<float4*>(dst) = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                                                  __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
    *reinterpret_cast<float4*>(dst + 4) = make_float4(__uint_as_float(u.z << 16), __uint_as_float(u.z & 0xFFFF0000u),
                                                      __uint_as_float(u.w << 16), __uint_as_float(u.w & 0xFFFF0000u));
  }
};

template <int NT, typename TIN, typename TOUT>
__global__ __launch_bounds__(threads_of<NT>(), NT == 1 ? 2 : 1) void prefill_small_kernel(const TIN* __restrict__ q, const TIN* __restrict__ k,
                                                            const TIN* __restrict__ v, TOUT* __restrict__ o,
                                                            float* __restrict__ state, size_t t_base,
                                                            int* __restrict__ sync, float* __restrict__ imgs, int N,
                                                            int nseg, int G, float inv_a, int wait_limit) {
  constexpr int kWaves = waves_of<NT>(), kThreads = threads_of<NT>(), kL = seg_tokens<NT>();
  using I = Img<NT>;
  constexpr int IMG = I::kFloats, NV = I::kPer;
  __shared__ __align__(16) float Xq[kL][kQS];
  __shared__ __align__(16) float Xk[kL][kQS];
  __shared__ __align__(16) float Xv[kL][kVS];
  __shared__ __align__(16) float W[kWaves][IMG];  // the waves' sums
  __shared__ __align__(16) float Pc[IMG];    // the segment's exclusive prefix
  __shared__ int s_ticket;

  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int ticket = blockIdx.x;
  if (sync != nullptr) {  // uniform
    // the sequence (XCD-affine); its counter gives the segment
    const int b = sequence_of_workgroup(blockIdx.x, nseg, gridDim.x / nseg);
    if (tid == 0)
      s_ticket = b * nseg + __hip_atomic_fetch_add(&sync[kHdr + (size_t)b * nseg + nseg - 1], 1, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    ticket = __builtin_amdgcn_readfirstlane(s_ticket);
  }
  const int bh = ticket / nseg, seg = ticket % nseg;
  const int nvalid = min(kL, N - seg * kL);
  const size_t row0 = (size_t)bh * N + (size_t)seg * kL;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  // ---- 1. the segment into LDS (every 16-byte load issued before any store),
  // and the caller's state into registers (thread t holds image units t,
  // t + kThreads, ...).  Every segment reads the caller's state here; each one
  // publishes in step 3 only after these reads have returned, and the final
  // state is written in step 7 only by a segment that has seen every earlier
  // segment publish, so the reads never race with that write.
  f32x4 cst[NV];
  {
    constexpr int P = Raw<TIN>::kPer;
    constexpr int QI = kL * kD / P / kThreads, VI = kL * kDV / P / kThreads;  // units per thread
    u32x4 xq[QI], xk[QI], xv[VI];
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < QI; ++i) {
      const int u = tid + kThreads * i, r = u / (kD / P), c = (u % (kD / P)) * P;
      xq[i] = r < nvalid ? *reinterpret_cast<const u32x4*>(q + (row0 + r) * kD + c) : z;
      xk[i] = r < nvalid ? *reinterpret_cast<const u32x4*>(k + (row0 + r) * kD + c) : z;
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int u = tid + kThreads * i, r = u / (kDV / P), c = (u % (kDV / P)) * P;
      xv[i] = r < nvalid ? *reinterpret_cast<const u32x4*>(v + (row0 + r) * kDV + c) : z;
    }
#pragma unroll
    for (int i = 0; i < NV; ++i)
      cst[i] = tid + kThreads * i < I::kVec ? state_unit_load<NT>(state, t_base, bh, tid + kThreads * i) : zero;
#pragma unroll
    for (int i = 0; i < QI; ++i) {
      const int u = tid + kThreads * i, r = u / (kD / P), c = (u % (kD / P)) * P;
      Raw<TIN>::put(&Xq[r][c], xq[i]);
      Raw<TIN>::put(&Xk[r][c], xk[i]);
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int u = tid + kThreads * i, r = u / (kDV / P), c = (u % (kDV / P)) * P;
      Raw<TIN>::put(&Xv[r][c], xv[i]);
    }
  }
  __syncthreads();

  // ---- 2. wave w's sum over tokens 32w .. 32w+31 (lane (li, g) takes keys
  // 4s + g); h0 keeps M's part from the wave's first 16 tokens (its first chunk)
  f32x4 h0[4];
  {
    const int t0 = 32 * w;
    f32x4 m[4] = {zero, zero, zero, zero};
    float cs[4] = {0.f, 0.f, 0.f, 0.f}, ks = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int key = t0 + 4 * s + g;
      const float kv = Xk[key][li];
      ks += kv;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const float vv = Xv[key][16 * ct + li];
        cs[ct] += vv;
        if constexpr (NT == 2) m[ct] = mfma_f32_k4(kv, vv, m[ct]);  // M[dim][col] += k[key][dim] v[key][col]
      }
      if (s == 3) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) h0[ct] = m[ct];
      }
    }
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      ks += __shfl_xor(ks, off);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) cs[ct] += __shfl_xor(cs[ct], off);
    }
    float* Wi = W[w];
    if constexpr (NT == 2) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) Wi[kDV + (4 * g + r) * kDV + 16 * ct + li] = m[ct][r];
    }
    if (g == 0) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) Wi[16 * ct + li] = cs[ct];
      if constexpr (NT == 2) Wi[I::kK + li] = ks;
    }
    if (lane == 0) Wi[I::kCnt] = (float)max(0, min(32, nvalid - t0));
    if (lane < IMG - I::kPad) Wi[I::kPad + lane] = 0.0f;
  }
  __syncthreads();

  // ---- 3. the segment's sum (agg), published at once (flag 1) unless no
  // segment reads it (a group leader's, the last segment's).  Images and flags
  // never include the caller's state.
  // W[w] becomes the sum of the waves before w (wave w's starting point in
  // step 4); each thread rewrites only the units it reads.
  f32x4 agg[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int f = 4 * min(tid + kThreads * i, I::kVec - 1);
    f32x4 x[kWaves];
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) x[ww] = *reinterpret_cast<const f32x4*>(&W[ww][f]);
    __syncthreads();  // every thread has read its units (the clamped last unit is read twice)
    f32x4 run = zero;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      if (tid + kThreads * i < I::kVec) *reinterpret_cast<f32x4*>(&W[ww][f]) = run;
      run += x[ww];
    }
    agg[i] = run;
  }
  __syncthreads();
  const size_t head0 = (size_t)bh * nseg;
  auto flag_of = [&](int j) { return &sync[kHdr + head0 + j]; };
  auto img_of = [&](int j, int total) { return imgs + ((head0 + j) * 2 + total) * IMG; };
  // groups of G consecutive segments; the last member of a group that has a
  // later group (its leader) publishes the group's total instead of its sum
  const int grp = seg / G, ing = seg % G;
  const bool leader = ing == G - 1 && seg < nseg - 1;
  auto store_img = [&](float* dst, const f32x4(&x)[NV]) {
    const __amdgpu_buffer_rsrc_t r = rsrc(dst, IMG);
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (tid + kThreads * i < I::kVec)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x[i]), r, (tid + kThreads * i) * 16, 0,
                                               kSC1);
  };
  if (sync != nullptr && !leader && seg < nseg - 1) {  // uniform
    store_img(img_of(seg, 0), agg);
    raise_flag(flag_of(seg), 1);
  }

  // ---- 4. local replay, while the earlier segments publish: wave w starts
  // from the earlier waves' sums alone.  Lane (li, g) holds C[16 ct + li],
  // K[li] and the count, and ends with y[c][ct][r] = Y[token 4g + r of chunk
  // c][column 16 ct + li] and den[c] = normaliser of token li of chunk c, both
  // without the prefix and without the (Q / a) M term of Y; Ms[c][ct][r] =
  // M[4g + r][16 ct + li] at the start of chunk c (an MFMA accumulator tile),
  // whose term is added in step 6 together with the prefix's.
  f32x4 y[2][4], Ms[2][4];
  float den[2];
  {
    float C[4], Kd = 0.f, cnt;
    auto start = [&](int f) { return W[w][f]; };  // the earlier waves' sums
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      C[ct] = start(16 * ct + li);
      Ms[0][ct] = zero;
      if constexpr (NT == 2) {
#pragma unroll
        for (int r = 0; r < 4; ++r) Ms[0][ct][r] = start(kDV + (4 * g + r) * kDV + 16 * ct + li);
      }
      Ms[1][ct] = Ms[0][ct] + h0[ct];
    }
    if constexpr (NT == 2) Kd = start(I::kK + li);
    cnt = start(I::kCnt);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int t0 = 32 * w + 16 * c;  // first token of the chunk in the segment
      // P[token li][key 4g + r] (MFMA with A = k rows, B = q rows gives D[key][token])
      float p[4];
      if constexpr (NT == 2) {
        f32x4 sc = zero;
#pragma unroll
        for (int st = 0; st < 4; ++st) sc = mfma_f32_k4(Xk[t0 + li][4 * st + g], Xq[t0 + li][4 * st + g], sc);
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = 4 * g + r <= li ? fmaf(sc[r], inv_a, 1.0f) : 0.0f;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = 4 * g + r <= li ? 1.0f : 0.0f;
      }
      float rs = (p[0] + p[1]) + (p[2] + p[3]);
      rs += __shfl_xor(rs, 16);
      rs += __shfl_xor(rs, 32);
      // value operands: in k-step st, k-slot g is key 4g + st
      float vb[4][4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int st = 0; st < 4; ++st) vb[ct][st] = Xv[t0 + 4 * g + st][16 * ct + li];
      // Y = C + P V
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        f32x4 acc = {C[ct], C[ct], C[ct], C[ct]};
#pragma unroll
        for (int st = 0; st < 4; ++st) acc = mfma_f32_k4(p[st], vb[ct][st], acc);
        y[c][ct] = acc;
      }
      // normaliser of token li: count + row sum of P + (q / a) . K
      den[c] = cnt + rs;
      if constexpr (NT == 2) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) part += Xq[t0 + li][4 * g + e] * inv_a * __shfl(Kd, 4 * g + e);
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        den[c] += part;
      }
      if (c == 1) break;  // the state after the last chunk is not needed
      // C, K and the count take the chunk (rows past the end of the sequence
      // are zero); M's part is h0
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        float cs = (vb[ct][0] + vb[ct][1]) + (vb[ct][2] + vb[ct][3]);
        cs += __shfl_xor(cs, 16);
        cs += __shfl_xor(cs, 32);
        C[ct] += cs;
      }
      if constexpr (NT == 2) {
        float ksum = 0.f;
#pragma unroll
        for (int st = 0; st < 4; ++st) ksum += Xk[t0 + 4 * g + st][li];
        ksum += __shfl_xor(ksum, 16);
        ksum += __shfl_xor(ksum, 32);
        Kd += ksum;
      }
      cnt += (float)max(0, min(16, nvalid - t0));
    }
  }

  // ---- 5. the sum of the earlier segments (look; zero for segment 0), then the
  // segment's exclusive prefix pre = caller's state + look.  Segment s = G grp +
  // ing adds (A) the sums of segments G grp .. s - 1 of its own group and (B) the
  // totals of groups 0 .. grp - 1, always these images and in this order, so
  // the result does not depend on timing.  A leader publishes its group's total
  // (A + its own sum, flag 2) between the two.
  f32x4 look[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) look[i] = zero;
  if (sync != nullptr && seg > 0) {  // uniform
    // Wave 0 waits until segments `slot(k)`, k in [0, m), show flag >= need
    // (64 flags per read: consecutive segments have consecutive flag words);
    // then every wave is released by the barrier.
    auto wait_all = [&](int m, int need, auto slot) {
      if (w == 0) {
        for (int k0 = 0; k0 < m; k0 += 64) {
          const int k = k0 + lane;
          int it = 0;
          for (; it < wait_limit; ++it) {
            const int f = k < m ? __hip_atomic_load(flag_of(slot(k)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                : need;
            if (__ballot(f < need) == 0) break;
            __builtin_amdgcn_s_sleep(4);
          }
          if (it == wait_limit && lane == 0)  // ran out: the results are wrong, and the header says so
            __hip_atomic_store(&sync[1], kN3ErrTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __syncthreads();  // also: every wave is done with Xv before it is reused below
    };
    // sum of images `img(k)`, k in [0, m): shared out over the waves, wave w
    // taking images w, w + kWaves, ...; each lane sums 16-byte units lane,
    // lane + 64, ... of its wave's images (BI images' loads in flight at a time;
    // a load past the image or past the last image reads an empty buffer
    // range, i.e. zeros).  The waves' partial sums meet in LDS (in the v buffer)
    // and are added in wave order.
    auto sum_images = [&](int m, auto img, f32x4(&out)[NV]) {
      constexpr int U = (I::kVec + 63) / 64, BI = NT == 2 ? 2 : 4;
      f32x4 part[U];
#pragma unroll
      for (int u = 0; u < U; ++u) part[u] = zero;
      for (int i0 = w; i0 < m; i0 += kWaves * BI) {  // uniform
        f32x4 x[BI][U];
#pragma unroll
        for (int b = 0; b < BI; ++b) {
          const int i = i0 + kWaves * b;
          const __amdgpu_buffer_rsrc_t r = rsrc(i < m ? img(i) : imgs, i < m ? IMG : 0);
#pragma unroll
          for (int u = 0; u < U; ++u)
            x[b][u] =
                __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (lane + 64 * u) * 16, 0, kSC1));
        }
#pragma unroll
        for (int b = 0; b < BI; ++b)
#pragma unroll
          for (int u = 0; u < U; ++u) part[u] += x[b][u];
      }
      f32x4* red = reinterpret_cast<f32x4*>(&Xv[0][0]);  // [kWaves][kVec]
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (lane + 64 * u < I::kVec) red[w * I::kVec + lane + 64 * u] = part[u];
      __syncthreads();
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = min(tid + kThreads * i, I::kVec - 1);
        out[i] = red[e];
#pragma unroll
        for (int ww = 1; ww < kWaves; ++ww) out[i] += red[ww * I::kVec + e];
      }
    };
    const int g0 = grp * G;
    if (ing > 0) {  // uniform: (A)
      wait_all(ing, 1, [&](int k) { return g0 + k; });
      sum_images(ing, [&](int k) { return img_of(g0 + k, 0); }, look);
    }
    if (leader) {  // uniform
      f32x4 x[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) x[i] = look[i] + agg[i];
      store_img(img_of(seg, 1), x);
      raise_flag(flag_of(seg), 2);
    }
    if (grp > 0) {  // uniform: (B)
      f32x4 tot[NV];
      wait_all(grp, 2, [&](int k) { return k * G + G - 1; });
      sum_images(grp, [&](int k) { return img_of(k * G + G - 1, 1); }, tot);
#pragma unroll
      for (int i = 0; i < NV; ++i) look[i] = tot[i] + look[i];
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (tid + kThreads * i < I::kVec) *reinterpret_cast<f32x4*>(&Pc[4 * (tid + kThreads * i)]) = cst[i] + look[i];
  __syncthreads();

  // ---- 6. the prefix's part of every output (C, count + (Q / a) . K) and the
  // (Q / a) M term with M = the prefix's + the chunk's local start; o = Y / den,
  // staged through LDS (wave w's own rows of the v buffer) so that every lane
  // stores 16 contiguous bytes, as streaming (nontemporal) stores: the outputs
  // are not read again here
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int t0 = 32 * w + 16 * c;
    float qa[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) qa[e] = Xq[t0 + li][4 * g + e] * inv_a;
    float dn = den[c] + Pc[I::kCnt];
    if constexpr (NT == 2) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) part += qa[e] * Pc[I::kK + 4 * g + e];
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      dn += part;
    }
    float inv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) inv[r] = 1.0f / __shfl(dn, 4 * g + r);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const float cp = Pc[16 * ct + li];
      f32x4 acc = y[c][ct] + f32x4{cp, cp, cp, cp};
      if constexpr (NT == 2) {
#pragma unroll
        for (int st = 0; st < 4; ++st)
          acc = mfma_f32_k4(qa[st], Pc[kDV + (4 * g + st) * kDV + 16 * ct + li] + Ms[c][ct][st], acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) Xv[t0 + 4 * g + r][16 * ct + li] = acc[r] * inv[r];
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if constexpr (std::is_same<TOUT, float>::value) {
#pragma unroll
    for (int it = 0; it < 8; ++it) {  // rows 4 it + g, 16-byte unit li
      const int row = 32 * w + 4 * it + g;
      if (row < nvalid)
        __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(&Xv[row][4 * li]),
                                    reinterpret_cast<f32x4*>(o + (row0 + row) * kDV + 4 * li));
    }
  } else {
#pragma unroll
    for (int it = 0; it < 4; ++it) {  // rows 8 it + lane / 8, 8 values from column 8 (lane % 8)
      const int row = 32 * w + 8 * it + (lane >> 3), c0 = 8 * (lane & 7);
      if (row < nvalid) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(&Xv[row][c0]);
        const f32x4 b = *reinterpret_cast<const f32x4*>(&Xv[row][c0 + 4]);
        u32x4 u;
        u.x = __builtin_bit_cast(uint32_t, bf16x2{f32_to_bf16(a[0]), f32_to_bf16(a[1])});
        u.y = __builtin_bit_cast(uint32_t, bf16x2{f32_to_bf16(a[2]), f32_to_bf16(a[3])});
        u.z = __builtin_bit_cast(uint32_t, bf16x2{f32_to_bf16(b[0]), f32_to_bf16(b[1])});
        u.w = __builtin_bit_cast(uint32_t, bf16x2{f32_to_bf16(b[2]), f32_to_bf16(b[3])});
        __builtin_nontemporal_store(u, reinterpret_cast<u32x4*>(o + (row0 + row) * kDV + c0));
      }
    }
  }

  // ---- 7. the last segment writes the final state: caller's + earlier + own
  if (seg == nseg - 1) {  // uniform
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (tid + kThreads * i < I::kVec)
        state_unit_store<NT>(state, t_base, bh, tid + kThreads * i, cst[i] + look[i] + agg[i]);
  }
}

// Zeroes the error code and every flag word (the ticket counters among them),
// and sets the header's magic word (which tells taylor_prefill_check that the
// error word is live).
static __global__ void clear_kernel(int* sync, int nslots) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nslots) sync[kHdr + i] = 0;
  if (i < 3) sync[i] = i == 2 ? kN3Magic : 0;
}

// Flag words per call, rounded up so that the images start 256-byte aligned.
inline size_t flag_words(int BH, int nseg) { return ((size_t)BH * nseg + 63) / 64 * 64; }

// Group size of the prefix over nseg segments: one group (every segment adds
// the sums of all earlier ones) up to 32 segments, else about sqrt(nseg), so
// that no segment adds more than about 2 sqrt(nseg) images.
inline int group_size(int nseg) {
  if (nseg <= 32) return nseg;
  int G = 1;
  while (G * G < nseg) ++G;
  return G;
}

template <int NT, typename TIN, typename TOUT>
hipError_t launch_t(const PrefillArgs& a) {
  constexpr int kL = seg_tokens<NT>(), kThreads = threads_of<NT>();
  const int nseg = (a.N + kL - 1) / kL;
  const size_t t_base = (size_t)a.BH * state_width(NT) * kDV;
  int* sync = nullptr;
  float* imgs = nullptr;
  hipEvent_t* ev = a.events;
  if (ev) (void)hipEventRecord(ev[0], a.stream);
  if (nseg > 1) {
    const int nslots = a.BH * nseg;
    sync = reinterpret_cast<int*>(a.workspace);
    imgs = a.workspace + kHdr + flag_words(a.BH, nseg);
    hipLaunchKernelGGL(clear_kernel, dim3((nslots + 255) / 256), dim3(256), 0, a.stream, sync, nslots);
  }
  if (ev) {
    // events 2 and 3 are recorded by the dispatch itself, at the kernel's
    // start and end (no launch gap inside the interval)
    (void)hipEventRecord(ev[1], a.stream);
    hipExtLaunchKernelGGL((prefill_small_kernel<NT, TIN, TOUT>), dim3(a.BH * nseg), dim3(kThreads), 0, a.stream,
                          ev[2], ev[3], 0, static_cast<const TIN*>(a.q), static_cast<const TIN*>(a.k),
                          static_cast<const TIN*>(a.v), static_cast<TOUT*>(a.o), a.state, t_base, sync, imgs, a.N, nseg,
                          group_size(nseg), 1.0f / a.a, a.wait_limit);
  } else {
    hipLaunchKernelGGL((prefill_small_kernel<NT, TIN, TOUT>), dim3(a.BH * nseg), dim3(kThreads), 0, a.stream,
                       static_cast<const TIN*>(a.q), static_cast<const TIN*>(a.k), static_cast<const TIN*>(a.v),
                       static_cast<TOUT*>(a.o), a.state, t_base, sync, imgs, a.N, nseg, group_size(nseg), 1.0f / a.a,
                       a.wait_limit);
  }
  return hipGetLastError();
}

template <int NT>
hipError_t launch_n(const PrefillArgs& a) {
  if (a.in_bf16) return a.out_bf16 ? launch_t<NT, uint16_t, uint16_t>(a) : launch_t<NT, uint16_t, float>(a);
  return a.out_bf16 ? launch_t<NT, float, uint16_t>(a) : launch_t<NT, float, float>(a);
}

}  // namespace small

size_t prefill_small_workspace_floats(int BH, int N, int n) {
  const int L = n == 2 ? small::seg_tokens<2>() : small::seg_tokens<1>();
  const int nseg = (N + L - 1) / L;
  if (BH <= 0 || nseg <= 1) return 0;
  const size_t img = n == 2 ? small::Img<2>::kFloats : small::Img<1>::kFloats;
  const size_t slots = (size_t)BH * nseg;
  return small::kHdr + small::flag_words(BH, nseg) + slots * 2 * img;
}

hipError_t launch_prefill_small(const PrefillArgs& a) {
  return a.n == 2 ? small::launch_n<2>(a) : small::launch_n<1>(a);
}

}  // namespace taylor
