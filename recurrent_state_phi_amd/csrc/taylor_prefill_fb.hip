// Chunked prefill for n = 4, 5, 6 at d = 16 and n = 1, 2, 3 at d = 32, 64
// (section 3.5 of "A Taylor-Series Route to
// Linear-Time Transformers with a Fixed Number of Recurrent States",
// arXiv 2610.20637), where the stacked state has D = 969, 4,845 or 20,349
// rows of d_v + 1 = 65 floats (252 KB, 1.26 MB, 5.3 MB per head): more than
// one workgroup can hold in registers or LDS.
//
// The feature rows are therefore split into NFB blocks of 11 tiles (176 rows;
// 6, 28 or 116 blocks).
// Everything the method does is linear in the state rows, so each block is an
// independent problem:
//   * segment sums, scan and replay run per (head, segment, feature block),
//     exactly as in the unblocked kernels (the scan works on rows, so it is
//     shared);
//   * the replay of block fb writes the block's share of the unnormalised
//     outputs, Y_fb = phi_hat(Q)_fb S_fb (+ the masked diagonal block P [V, 1]
//     for fb = 0), to a workspace; a combine kernel then forms
//     o = sum_fb Y_fb[:d_v] / sum_fb Y_fb[d_v]  (Eq. (5)).
// Arithmetic is float32 throughout (16x16x4 float32 MFMA); bfloat16 inputs are
// widened when staged.  Feature rows follow the caller's layout (m ascending,
// lexicographic multi-indices, sqrt-multinomial weights) and come from a table
// (orders up to 3 for n = 4, up to 5 for n = 5, 6).
//
// Work inside one 256-thread workgroup (4 waves): wave w owns value columns
// 16w..16w+15 of the block's state (11 accumulator tiles), read and updated on
// MFMA.  The ones-column T of the block (176 floats) is spread over the
// threads, one row each, and its read (a dot product of the query features
// with T, plus the row sums of P for block 0) and update (column sums of the
// key features) are plain sums over all 256 threads, so every wave does the
// same matrix work.
// Per chunk: stage q, k, v and T | features of the block and (fb = 0) the
// masked polynomial block P into LDS | state read and update.  Thread
// fl < 176 owns row F0 + fl of the block for the whole kernel: it decodes the
// row's table entry once (coordinates, weight, alpha_m) and forms that row's
// feature for every token of every chunk as weight * x_i1 * ... * x_i(n-1),
// unused coordinate slots pointing at a column that holds 1.  The next
// chunk's q, k, v are loaded into registers while the current one is
// computed.
#include <type_traits>

#include "taylor_device.h"
#include "taylor_launch.h"

namespace taylor {
namespace fb {

constexpr int kFT = 11;                      // feature tiles per block
constexpr int kBF = 16 * kFT;                // 176 rows per block
constexpr int kPS = kBF + 4;                 // feature row stride in LDS (16-byte aligned rows)
constexpr int kYS = kDV + 4;                 // partial-output row: 64 values, the normaliser, padding
// Feature blocks of the state: d = 16: 6, 28, 116 for n = 4, 5, 6;
// d = 32: 1, 1, 4 and d = 64: 1, 1, 13 for n = 1, 2, 3.
constexpr int blocks_of(int d, int n) { return (state_width_d(d, n) + kBF - 1) / kBF; }

__constant__ FeatureTable kTab = make_feature_table();                 // d = 16, n = 4 (orders <= 3)
static __device__ RowTable<16, 5> kTab16 = make_row_table<16, 5>();   // d = 16, n = 5, 6
static __device__ RowTable<32, 2> kTab32 = make_row_table<32, 2>();   // d = 32, n <= 3
static __device__ RowTable<64, 2> kTab64 = make_row_table<64, 2>();   // d = 64, n <= 3

// The row table a (KD, NT) kernel reads (all but d = 16, n = 4).
template <int KD>
__device__ __forceinline__ uint32_t row_code(int f) {
  if constexpr (KD == 16) return kTab16.code[f];
  else if constexpr (KD == 32) return kTab32.code[f];
  else return kTab64.code[f];
}
template <int KD> constexpr int table_orders() { return KD == 16 ? 5 : 2; }

template <int C, int KD>
struct Lds {
  float Xq[C][KD + 1];  // column KD: 1 (the factor of unused coordinate slots)
  float Xk[C][KD + 1];  // column KD: 1, or 0 for a padding token
  float VT[kDV][C + 4];  // V transposed (token index fastest; 16-byte aligned rows)
  float PhQ[C][kPS];
  float PhKT[kBF][C + 4];  // key features, feature-major (token index fastest)
  float P[C][C + 4];
  float Ts[kBF];
  float Yd[C];  // normaliser of each token (single-block states only)
};

template <typename IT> __device__ __forceinline__ float ld(const IT* p, size_t i) { return Elem<IT>::load(p, i); }

// p_4(y) = 1 + y + y^2/2 + y^3/6
__device__ __forceinline__ float poly4(float y) { return 1.0f + y * (1.0f + y * (0.5f + y * (1.0f / 6.0f))); }
// p_n(y) = sum_{m<n} y^m / m! by Horner's rule: 1 + y (1 + y/2 (1 + y/3 (...))).
template <int NT>
__device__ __forceinline__ float poly(float y) {
  if constexpr (NT == 4) return poly4(y);
  float r = 1.0f;
#pragma unroll
  for (int m = NT - 1; m >= 1; --m) r = 1.0f + y * r * (1.0f / (float)m);
  return r;
}

template <int NT, int KD, int C, bool FULL, typename IT, typename TOUT>
__global__ __launch_bounds__(256, C == 32 ? 2 : 1) void prefill_fb_kernel(const IT* __restrict__ q, const IT* __restrict__ k,
                                                         const IT* __restrict__ v, float* __restrict__ Yp,
                                                         TOUT* __restrict__ o,
                                                         const float* __restrict__ pre_S,
                                                         const float* __restrict__ pre_T, int pre_slots,
                                                         float* __restrict__ dst_S, float* __restrict__ dst_T,
                                                         int dst_slots, int BH, int N, int nseg, int cps,
                                                         float inv_a) {
  __shared__ __align__(16) Lds<C, KD> L;
  constexpr int NTT = C / 16;
  constexpr int kD4 = state_width_d(KD, NT);  // rows of the stacked state
  constexpr int kNFB = blocks_of(KD, NT);
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: guards MFMAs
  const int fbk = blockIdx.x % kNFB;
  const int rest = blockIdx.x / kNFB;
  const int gseg = FULL ? nseg : nseg - 1;
  const int bh = rest / gseg, seg = rest % gseg;
  const int F0 = fbk * kBF;
  const int t_begin = seg * cps * C;
  const int t_end = min(N, t_begin + cps * C);
  const int col = 16 * w + li;

  // ---- the segment's starting state (rows F0 .. F0 + 175 of the block);
  //      thread tid < 176 holds T of row F0 + tid
  f32x4 Sacc[kFT];
  float treg = 0.0f;
  {
    const size_t slot = (size_t)bh * pre_slots + (pre_slots == 1 ? 0 : seg);
    const float* ps = (FULL && pre_S) ? pre_S + slot * kD4 * kDV : nullptr;
    const float* pt = (FULL && pre_T) ? pre_T + slot * kD4 : nullptr;
#pragma unroll
    for (int ft = 0; ft < kFT; ++ft)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = F0 + 16 * ft + 4 * g + r;
        Sacc[ft][r] = ps ? ps[(size_t)min(row, kD4 - 1) * kDV + col] : 0.0f;
        if (row >= kD4) Sacc[ft][r] = 0.0f;
      }
    if (pt && tid < kBF && F0 + tid < kD4) treg = pt[F0 + tid];
  }

  // ---- this thread's feature items: (row fl of the block, quarter qt of the
  //      chunk's tokens), items t, t + 256, t + 512 of the 4 * 176, so all
  //      256 threads share the feature work; for each, the row's coordinates
  //      (KD = the column of ones for unused slots) and its key- and
  //      query-side weights, decoded once
  constexpr int NF = NT > 1 ? NT - 1 : 1;  // coordinate slots: orders up to n - 1
  constexpr int kItems = 4 * kBF;
  constexpr int NIT = (kItems + 255) / 256;
  int fidx[NIT][NF];
  float wk[NIT], wq[NIT];  // 0 for rows past the state
  int ifl[NIT], iqt[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int item = tid + 256 * it;
    ifl[it] = item % kBF;
    iqt[it] = item < kItems ? item / kBF : 4;  // 4: no item
    const int f = F0 + ifl[it];
    const bool valid = f < kD4;
    const int fr = valid ? f : 0;
    if constexpr (KD == 16 && NT == 4) {
      const uint32_t c = kTab.code[fr];
      const int m = c & 3;
      const float a2 = inv_a * inv_a;
      const float am = m == 0 ? 1.0f : m == 1 ? inv_a : m == 2 ? 0.5f * a2 : a2 * inv_a * (1.0f / 6.0f);
#pragma unroll
      for (int p = 0; p < NF; ++p) fidx[it][p] = p < m ? (int)((c >> (2 + 4 * p)) & 15) : KD;
      const float wt = kTab.weight[fr];
      wk[it] = valid ? wt : 0.0f;
      wq[it] = valid ? wt * am : 0.0f;
    } else {
      constexpr int MAXM = table_orders<KD>();
      const uint32_t c = row_code<KD>(fr);
      const int m = c & 7;
#pragma unroll
      for (int p = 0; p < NF; ++p) fidx[it][p] = p < m ? row_coord<KD, MAXM>(c, p) : KD;
      const float wt = row_weight<KD, MAXM>(c);
      wk[it] = valid ? wt : 0.0f;
      wq[it] = valid ? alpha_of(inv_a, c) * wt : 0.0f;
    }
  }

  // ---- loads of one chunk into registers (token indices clamped into the
  //      chunk; values of padding tokens are replaced when staged)
  constexpr int NLK = C * KD / 256, NLV = C * kDV / 256;
  float rk[NLK], rq[NLK], rv[NLV];
  auto fetch = [&](int t0n) {
    const int last = min(C, t_end - t0n) - 1;
    const size_t basen = (size_t)bh * N + t0n;
#pragma unroll
    for (int e = 0; e < NLK; ++e) {
      const int i = tid + 256 * e, tok = min(i / KD, last), j = i % KD;
      rk[e] = ld(k, (basen + tok) * KD + j);
      if (FULL) rq[e] = ld(q, (basen + tok) * KD + j);
    }
#pragma unroll
    for (int e = 0; e < NLV; ++e) {
      const int i = tid + 256 * e, tok = min(i / kDV, last), j = i % kDV;
      rv[e] = ld(v, (basen + tok) * kDV + j);
    }
  };
  if (t_begin < t_end) fetch(t_begin);  // uniform

  for (int t0 = t_begin; t0 < t_end; t0 += C) {
    const int nv = min(C, t_end - t0);
    const size_t base = (size_t)bh * N + t0;

    // ---- stage q, k, v (float), zero for padding tokens; publish T of the block
#pragma unroll
    for (int e = 0; e < NLK; ++e) {
      const int i = tid + 256 * e, tok = i / KD, j = i % KD;
      L.Xk[tok][j] = tok < nv ? rk[e] : 0.0f;
      if (FULL) L.Xq[tok][j] = tok < nv ? rq[e] : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < NLV; ++e) {
      const int i = tid + 256 * e, tok = i / kDV, j = i % kDV;
      L.VT[j][tok] = tok < nv ? rv[e] : 0.0f;
    }
    if (tid < C) {
      L.Xk[tid][KD] = tid < nv ? 1.0f : 0.0f;  // the constant feature of a padding token is 0
      if (FULL) L.Xq[tid][KD] = 1.0f;
    }
    if (FULL && tid < kBF) L.Ts[tid] = treg;
    if (t0 + C < t_end) fetch(t0 + C);  // uniform
    __syncthreads();

    // ---- features of the block (query side scaled by alpha_m), and P for block 0
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      if (iqt[it] < 4) {
        const int fl = ifl[it];
#pragma unroll
        for (int i = 0; i < C / 4; ++i) {
          const int tok = iqt[it] * (C / 4) + i;
          float fk = wk[it], fq = wq[it];
#pragma unroll
          for (int p = 0; p < NF; ++p) {
            fk *= L.Xk[tok][fidx[it][p]];
            if (FULL) fq *= L.Xq[tok][fidx[it][p]];
          }
          L.PhKT[fl][tok] = fk;
          if (FULL) L.PhQ[tok][fl] = fq;
        }
      }
    }
    if (FULL && fbk == 0) {  // uniform
      // scores Q K^T on the matrix cores, one 16x16 tile per wave at a time;
      // the lane holds S[16a + 4g + r][16b + li]
      for (int tile = w; tile < NTT * NTT; tile += 4) {
        const int ta = tile / NTT, tb = tile % NTT;
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s4 = 0; s4 < KD / 4; ++s4)
          sc = mfma_f32_k4(L.Xq[16 * ta + li][4 * s4 + g], L.Xk[16 * tb + li][4 * s4 + g], sc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tq = 16 * ta + 4 * g + r, tk = 16 * tb + li;
          L.P[tq][tk] = tk <= tq ? poly<NT>(sc[r] * inv_a) : 0.0f;
        }
      }
    }
    __syncthreads();

    // ---- this block's share of the outputs: Y = phi_hat(Q)_fb S_fb (+ P [V, 1]).
    //      A state that fits one block (n = 3 at d = 16, n <= 2 at d = 32, 64)
    //      writes o = Y[:d_v] / Y[d_v] directly; otherwise the block's share of
    //      the unnormalised outputs goes to the workspace for the combine pass.
    //      With several feature blocks, the products below run at raised wave
    //      priority: the two workgroups of a CU are then mostly in different
    //      phases, and the one in its matrix phase issues first.
    if constexpr (kNFB > 1) __builtin_amdgcn_s_setprio(1);
    if constexpr (FULL) {
      // the block's share of the normaliser first: phi_hat(q)_fb . T_fb, plus
      // the row sum of P for block 0; 256 / C consecutive threads per token
      constexpr int TPT = 256 / C;
      {
        const int tok = tid / TPT, part = tid % TPT;
        float yd = 0.0f;
        for (int fl = part; fl < kBF; fl += TPT) yd += L.PhQ[tok][fl] * L.Ts[fl];
        if (fbk == 0) {  // uniform
          for (int tk = part; tk < C; tk += TPT) yd += L.P[tok][tk];
        }
#pragma unroll
        for (int off = 1; off < TPT; off <<= 1) yd += __shfl_xor(yd, off);
        if (part == 0) {
          if constexpr (kNFB == 1) L.Yd[tok] = yd;
          else if (tok < nv) Yp[((size_t)fbk * BH * N + base + tok) * kYS + kDV] = yd;
        }
      }
      if constexpr (kNFB == 1) __syncthreads();
#pragma unroll
      for (int mt = 0; mt < NTT; ++mt) {
        const int tok = 16 * mt + li;
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ft = 0; ft < kFT; ++ft) {
          const f32x4 a4 = *reinterpret_cast<const f32x4*>(&L.PhQ[tok][16 * ft + 4 * g]);
#pragma unroll
          for (int r = 0; r < 4; ++r) y = mfma_f32_k4(a4[r], Sacc[ft][r], y);
        }
        if (fbk == 0) {  // uniform
          // k-slot order: lane group g takes tokens g C/4 .. g C/4 + C/4 - 1, so
          // its operands for four k-steps are 16 contiguous bytes
          for (int s4 = 0; s4 < C / 16; ++s4) {
            const int k0 = g * (C / 4) + 4 * s4;
            const f32x4 a4 = *reinterpret_cast<const f32x4*>(&L.P[tok][k0]);
            const f32x4 b4 = *reinterpret_cast<const f32x4*>(&L.VT[col][k0]);
#pragma unroll
            for (int r = 0; r < 4; ++r) y = mfma_f32_k4(a4[r], b4[r], y);
          }
        }
        // lane holds Y[token 16mt + 4g + r][col]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * mt + 4 * g + r;
          if (t < nv) {
            if constexpr (kNFB == 1) Elem<TOUT>::store(o, (base + t) * kDV + col, y[r] / L.Yd[t]);
            else Yp[((size_t)fbk * BH * N + base + t) * kYS + col] = y[r];
          }
        }
      }
    }

    // ---- state update: S_fb += phi(K)_fb^T V (MFMA), T_fb += phi(K)_fb^T 1
    //      (padding tokens have zero features, the constant one included)
    //      k-slot order as in the diagonal block: lane group g takes tokens
    //      g C/4 .. g C/4 + C/4 - 1, four k-steps per 16-byte read
    for (int s4 = 0; s4 < C / 16; ++s4) {
      const int k0 = g * (C / 4) + 4 * s4;
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(&L.VT[col][k0]);
#pragma unroll
      for (int ft = 0; ft < kFT; ++ft) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(&L.PhKT[16 * ft + li][k0]);
#pragma unroll
        for (int r = 0; r < 4; ++r) Sacc[ft] = mfma_f32_k4(a4[r], b4[r], Sacc[ft]);
      }
    }
    if constexpr (kNFB > 1) __builtin_amdgcn_s_setprio(0);
    if (tid < kBF) {
      float ts = 0.0f;
#pragma unroll
      for (int t4 = 0; t4 < C; t4 += 4) {
        const f32x4 x4 = *reinterpret_cast<const f32x4*>(&L.PhKT[tid][t4]);
        ts += x4[0] + x4[1] + x4[2] + x4[3];
      }
      treg += ts;
    }
    __syncthreads();
  }

  // ---- write the block's rows of the state (last segment) or of the segment sum
  const bool write = FULL ? (seg == nseg - 1) : true;
  if (write) {
    const size_t slot = (size_t)bh * dst_slots + (dst_slots == 1 ? 0 : seg);
    float* ds = dst_S + slot * kD4 * kDV;
    float* dt = dst_T + slot * kD4;
#pragma unroll
    for (int ft = 0; ft < kFT; ++ft)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = F0 + 16 * ft + 4 * g + r;
        if (row < kD4) ds[(size_t)row * kDV + col] = Sacc[ft][r];
      }
    if (tid < kBF && F0 + tid < kD4) dt[F0 + tid] = treg;
  }
}

// o = sum over blocks of the numerators / sum of the normalisers (Eq. (5)).
// 16 threads per output row, 4 columns each (16-byte reads of the 68-float
// partial rows); the blocks are added in order.
template <int kNFB, typename TOUT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ Yp, TOUT* __restrict__ o,
                                                      size_t rows) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;  // (row, column quad)
  if (i >= rows * (kDV / 4)) return;
  const size_t row = i / (kDV / 4);
  const int c4 = (int)(i % (kDV / 4));
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  float den = 0.0f;
#pragma unroll 4
  for (int b = 0; b < kNFB; ++b) {
    const float* y = Yp + ((size_t)b * rows + row) * kYS;
    num += *reinterpret_cast<const f32x4*>(y + 4 * c4);
    den += y[kDV];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) Elem<TOUT>::store(o, row * kDV + 4 * c4 + e, num[e] / den);
}

template <int NT, int KD, int C, typename IT, typename TOUT>
hipError_t launch(const PrefillArgs& a) {
  constexpr int kD4 = state_width_d(KD, NT);
  constexpr int kNFB = blocks_of(KD, NT);
  const PrefillPlan& pl = a.plan;
  float* st_S = a.state;
  float* st_T = a.state + (size_t)a.BH * kD4 * kDV;
  const float inv_a = 1.0f / a.a;
  const IT* q = static_cast<const IT*>(a.q);
  const IT* k = static_cast<const IT*>(a.k);
  const IT* v = static_cast<const IT*>(a.v);
  // workspace: [segment sums / prefixes when nseg > 1][block outputs]
  // (rounded up to 4 floats, so the partial-output rows stay 16-byte aligned)
  const size_t agg = pl.nseg > 1 ? ((size_t)a.BH * pl.nseg * kD4 * (kDV + 1) + 3) / 4 * 4 : 0;
  float* W_S = a.workspace;
  float* W_T = a.workspace + (size_t)a.BH * pl.nseg * kD4 * kDV;
  float* Yp = a.workspace + agg;
  hipEvent_t* ev = a.events;
  if (ev) (void)hipEventRecord(ev[0], a.stream);
  if (pl.nseg > 1) {
    hipLaunchKernelGGL((prefill_fb_kernel<NT, KD, C, false, IT, TOUT>), dim3(a.BH * (pl.nseg - 1) * kNFB), dim3(256), 0,
                       a.stream, q, k, v, (float*)nullptr, (TOUT*)nullptr, (const float*)nullptr,
                       (const float*)nullptr, 1, W_S, W_T, pl.nseg, a.BH, a.N, pl.nseg, pl.chunks_per_seg, inv_a);
    if (ev) (void)hipEventRecord(ev[1], a.stream);
    if (hipError_t e = launch_segment_scan(st_S, st_T, W_S, W_T, kD4, pl.nseg, a.BH, a.stream)) return e;
    if (ev) (void)hipEventRecord(ev[2], a.stream);
    hipLaunchKernelGGL((prefill_fb_kernel<NT, KD, C, true, IT, TOUT>), dim3(a.BH * pl.nseg * kNFB), dim3(256), 0,
                       a.stream, q, k, v, Yp, static_cast<TOUT*>(a.o), W_S, W_T, pl.nseg, st_S, st_T, 1, a.BH, a.N,
                       pl.nseg, pl.chunks_per_seg, inv_a);
  } else {
    if (ev) {
      (void)hipEventRecord(ev[1], a.stream);
      (void)hipEventRecord(ev[2], a.stream);
    }
    hipLaunchKernelGGL((prefill_fb_kernel<NT, KD, C, true, IT, TOUT>), dim3(a.BH * kNFB), dim3(256), 0, a.stream, q, k,
                       v, Yp, static_cast<TOUT*>(a.o), st_S, st_T, 1, st_S, st_T, 1, a.BH, a.N, 1, pl.chunks_per_seg,
                       inv_a);
  }
  if constexpr (kNFB > 1) {
    const size_t rows = (size_t)a.BH * a.N;
    hipLaunchKernelGGL((combine_kernel<kNFB, TOUT>), dim3((unsigned)((rows * (kDV / 4) + 255) / 256)), dim3(256), 0,
                       a.stream,
                       Yp, static_cast<TOUT*>(a.o), rows);
  }
  if (ev) (void)hipEventRecord(ev[3], a.stream);
  return hipGetLastError();
}

template <int NT, int KD, int C>
hipError_t launch_c(const PrefillArgs& a) {
  if (a.in_bf16) return a.out_bf16 ? launch<NT, KD, C, uint16_t, uint16_t>(a) : launch<NT, KD, C, uint16_t, float>(a);
  return a.out_bf16 ? launch<NT, KD, C, float, uint16_t>(a) : launch<NT, KD, C, float, float>(a);
}

template <int NT, int KD>
hipError_t launch_n(const PrefillArgs& a) {
  switch (a.chunk) {
    case 32: return launch_c<NT, KD, 32>(a);
    case 64: return launch_c<NT, KD, 64>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace fb

int prefill_fb_blocks(int d, int n) { return fb::blocks_of(d, n); }

size_t prefill_fb_output_floats(int BH, int N, int d, int n) {
  const int nb = fb::blocks_of(d, n);
  return nb > 1 ? (size_t)nb * BH * N * fb::kYS : 0;  // one block writes o directly
}

hipError_t launch_prefill_fb(const PrefillArgs& a) {
  if (a.d == 16) {
    switch (a.n) {
      case 3: return fb::launch_n<3, 16>(a);
      case 4: return fb::launch_n<4, 16>(a);
      case 5: return fb::launch_n<5, 16>(a);
      case 6: return fb::launch_n<6, 16>(a);
    }
  } else if (a.d == 32 || a.d == 64) {
    switch (a.n) {
      case 1: return a.d == 32 ? fb::launch_n<1, 32>(a) : fb::launch_n<1, 64>(a);
      case 2: return a.d == 32 ? fb::launch_n<2, 32>(a) : fb::launch_n<2, 64>(a);
      case 3: return a.d == 32 ? fb::launch_n<3, 32>(a) : fb::launch_n<3, 64>(a);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace taylor
