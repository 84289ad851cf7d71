// Chunked prefill for n = 3 with bfloat16 q, k, v (section 3.5 of "A Taylor-Series
// Route to Linear-Time Transformers with a Fixed Number of Recurrent States",
// arXiv 2610.20637): float32 state, bfloat16 matrix-core operands, float32
// accumulation.
//
// ONE launch.  Every (b, h) sequence is cut into `nseg` segments; one
// workgroup per segment:
//
//  1. segment sum: the workgroup runs the state update over its segment from a
//     zero state (Eq. (6)-(7) summed over the segment; the states are additive
//     across chunks, section 3.5).  Segment 0 adds the caller's state to its
//     sum.  The sum A_s is published to the workspace.
//  2. prefix: the segments form groups of `gs` consecutive segments.  The last
//     segment of a group publishes the GROUP sum (its own sum plus those of
//     the earlier members) in place of its own.  The exclusive prefix of
//     segment s is then the group sums of the earlier groups plus the sums of
//     the earlier members of its own group: at most about 2 sqrt(nseg) state
//     images per workgroup, all published right after step 1.
//  3. replay: it runs the segment again from its prefix, producing the outputs
//     (Eq. (5)).  The last segment writes the final state (its prefix plus
//     its own sum) before its replay, so that the store is not left for the
//     end of the kernel; a single segment writes it after the replay.
//
// Every workgroup serves a fixed sequence (sequence_of_workgroup: all the
// segments of a sequence on one XCD where the dispatch allows) and takes its
// segment from that sequence's atomic ticket counter; a workgroup only ever
// waits for earlier segments of its own sequence, which hold smaller tickets
// of the same counter: they started before it, are running (or done), and
// every wait ends.  (One
// counter per sequence: a single counter for the whole grid serialises its
// atomics, about 12 ns each, so the last of 512 workgroups would start 6 us
// late.)
// Each wait is bounded all the same; a wait that runs out records an error
// code in the workspace.  The replay reads the segment's q, k, v shortly after
// step 1 read k and v, mostly from cache.
//
// Inside a chunk the work of the workgroup is split so that no feature value is
// computed twice and the large operands never make a round trip through LDS:
//
//  * The state read Y^T = S'^T phi'(Q)^T (the off-diagonal part of Eq. (5)) and
//    the diagonal block Y^T += [V, 1]^T P^T are split by TOKEN tile: wave w owns
//    tokens 16w..16w+15 (4 waves for 64-token chunks, 8 waves for 128-token
//    chunks, so that a 128-token workgroup, which fills most of the LDS on its
//    own, still keeps two waves on every SIMD).
//    The query features are built directly in the MFMA operand registers; the
//    score block Q K^T, the polynomial P and its row sums never leave registers.
//  * The state update S' += phi(K)^T [V, 1] (Eq. (6)-(7) summed over the chunk)
//    is split by FEATURE tile: with 4 waves, wave w owns tiles {w, w+4} for all
//    64 value columns and half of tile 8 + w/2; with 8 waves, tile w and a
//    quarter of tile 8 + w/4.  The key features are built in operand
//    registers from a transposed float32 copy of K; the ones-column T is the
//    same product against a ones operand, on the matrix cores as well.
//  * After its update every wave writes its part of the new state as a
//    bfloat16 copy of S'^T into LDS (double buffered) for the next chunk's read.
//    One barrier per chunk.
//
// Internal feature order ("R1"): 10 tiles of 16 rows.  Tile f < 8 holds the
// products x_r x_{(r+f) mod 16} for r = 0..15 (every unordered pair {i, j}
// exactly once: f is the forward distance j - i mod 16 when that is < 8);
// tile 8 holds x_r x_{r+8} for r < 8, then the constant feature (row 8) and
// seven zero rows; tile 9 holds the linear features x_r.  Internally the state
// rows are UNWEIGHTED sums of monomials; the sqrt-multinomial weight of
// section 3.4 appears squared (2 for i != j) on the query side instead, and is
// applied when the state is loaded from or stored to the caller's layout.
//
// The k-slot order of the state read pairs the tiles (0,2), (1,3), (4,6),
// (5,7), (8,9) into the five 32-wide k blocks; lane group g = 2*gh + h of the
// MFMA operand takes rows 8h..8h+7 of the gh-th tile of the pair.  With
// y = x rotated by 8h and z = x rotated by 8h + 2gh, the lane's 8 features of a
// k block are y_s z_{(s + d) mod 16} for compile-time s and d, so the query
// features need no runtime register indexing.
#include <hip/hip_ext.h>

#include <type_traits>

#include "taylor_device.h"
#include "taylor_launch.h"

namespace taylor {
namespace n3 {

constexpr int kD3 = 153;   // state rows in the caller's layout
constexpr int kNF = 160;   // internal feature rows (10 tiles)
constexpr int kSS = 168;   // row stride (bf16) of the S'^T copy (84 dwords: conflict-free 16-byte reads)
constexpr int kQS = 36;    // row stride (bf16) of the doubled q copy
constexpr int kKTRows = 16;

// Workspace of a multi-segment call (32-bit words):
//   [0]                    unused (zero)
//   [1]                    error code (kN3ErrTimeout: a wait ran out)
//   [2]                    kN3Magic (the flags below belong to this kernel)
//   [kHdr + kFlagStride * (b * nseg + s)]  flag of segment s of sequence b:
//                          nonzero once its image is published (one flag per
//                          256 bytes: polls of different flags do not queue
//                          on the same memory line); the last segment never
//                          publishes, and its slot counts the segments that
//                          have finished reading the caller's state;
//                          word kTicketWord of segment 0's slot is the
//                          sequence's ticket counter
//   then BH*nseg state images: the segment sums (group sums at the last
//   member of a group)
// The header (counter, error, flags) is cleared by a small kernel before every
// call.  A state image is the internal state in the register layout of the
// owning waves: kImgS floats of S' (every wave's (slot, column tile) pairs,
// lane-major, 16 bytes per lane) and 384 floats of T'.
constexpr int kHdr = 64;
constexpr int kFlagStride = 64;
constexpr int kTicketWord = 32;  // in the second 128-byte half of the slot, away from the flag word
constexpr int kImgS = 40 * 64 * 4;       // 40 owned (slot, column tile) pairs per workgroup
constexpr int kImgFloats = kImgS + 384;  // + T': waves x 3 slots x 4 lane groups x 4 rows (8 waves)

__host__ __device__ constexpr size_t header_words(int BH, int nseg) {
  return kHdr + (size_t)BH * nseg * kFlagStride;
}

// Waves of a workgroup: 4 for 64-token chunks, 8 for 128-token chunks.
template <int NW_>
struct Waves {
  static constexpr int NW = NW_;
  static constexpr int NTHREADS = 64 * NW;
  // feature-tile ownership (see Own)
  static constexpr bool HAS_S1 = NW == 4;
  static constexpr int NCT2 = NW == 4 ? 2 : 1;          // column tiles of slot 2
  static constexpr int NCTS = (HAS_S1 ? 8 : 4) + NCT2;  // owned (slot, column tile) pairs per wave
  static_assert(NW * NCTS == 40, "state image layout");
  static __device__ __forceinline__ constexpr bool has(int s, int ct) {
    return s == 0 || (s == 1 && HAS_S1) || (s == 2 && ct < NCT2);
  }
  static __device__ __forceinline__ constexpr int pair_index(int s, int ct) {
    return s == 0 ? ct : s == 1 ? 4 + ct : (HAS_S1 ? 8 : 4) + ct;
  }
};

// Chunk geometry of one pass (the segment-sum pass runs twice as many tokens
// per step as the replay).
template <int C, int NW>
struct Shape : Waves<NW> {
  static constexpr int NTT = C / 16;    // 16-token tiles per chunk
  static constexpr int NKB = C / 32;    // 32-token k blocks per chunk
  static constexpr int TPW = NTT / NW;  // token tiles per wave
  static constexpr int VS = C + 8;      // V^T row stride (bf16)
  static constexpr int KS = C + 4;      // K^T row stride (float)
  static_assert(TPW * NW == NTT, "token tiles per wave");
};

// LDS of the replay (every array double buffered by chunk parity).
template <int C>
struct Lds {
  alignas(16) uint16_t S[2][64][kSS];          // S'^T copy (bf16), k-slot order, swizzled
  alignas(16) uint16_t T[2][2][kNF];           // T' in k-slot order: bf16 high, low parts
  alignas(16) uint16_t V[2][64][C + 8];        // V^T (bf16), swizzled
  alignas(16) float K[2][kKTRows][C + 4];      // K^T (float)
  alignas(16) uint16_t Q[2][C][kQS];           // q twice per row: [x | x]
};

// The state of a workgroup in registers: 16x16 accumulator tiles of the owned
// (feature tile, column tile) pairs, and T' as column 0 of a 16x16 tile.
struct Acc {
  f32x4 s[3][4];
  f32x4 t[3];
};

__device__ __forceinline__ void zero_acc(Acc& a) {
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    a.t[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) a.s[s][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// 16-byte-chunk XOR swizzle of the rows of V^T: rows c and c + 16 land in
// different banks.
__device__ __forceinline__ int swz(int row, int e) { return (((e >> 3) ^ ((row >> 4) & 3)) << 3) | (e & 7); }

// k-slot of internal row rho of tile ft in the state read.
__device__ __forceinline__ int kslot_of(int ft, int rho) {
  int kb, gh;
  if (ft < 8) {
    kb = (ft >> 2) * 2 + (ft & 1);
    gh = (ft >> 1) & 1;
  } else {
    kb = 4;
    gh = ft - 8;
  }
  return 32 * kb + 8 * (2 * gh + (rho >> 3)) + (rho & 7);
}

// Row of the caller's layout (m ascending, lexicographic multi-indices) for
// internal row rho of tile ft, or -1 for a zero row; *w gets the
// sqrt-multinomial weight of that row.
// (Written with selects only: it is evaluated per lane next to global loads,
// which must not end up in divergent branches.)
__device__ __forceinline__ int abi_row(int ft, int rho, float* w) {
  const int j = ft < 8 ? ((rho + ft) & 15) : rho + 8;
  const int lo = rho < j ? rho : j, hi = rho < j ? j : rho;
  const int quad = 1 + kD + lo * kD - (lo * (lo - 1)) / 2 + (hi - lo);
  const bool pair = ft < 8 || (ft == 8 && rho < 8);
  *w = ft == 9 ? 1.0f : (pair ? (ft == 0 ? 1.0f : kSqrt2) : (rho == 8 ? 1.0f : 0.0f));
  return ft == 9 ? 1 + rho : (pair ? quad : (rho == 8 ? 0 : -1));
}

// Value of v held by lane (l + N) mod 16 of this lane's row of 16 lanes
// (DPP row rotation: row_ror by 16 - N).
template <int N>
__device__ __forceinline__ float from_lane_plus(float v) {
  static_assert(N > 0 && N < 16, "rotation");
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + (16 - N), 0xF, 0xF, false));
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const bf16x2 p = {f32_to_bf16(lo), f32_to_bf16(hi)};
  return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ float lo_f(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_f(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// Feature tiles and column tiles a wave owns.  4 waves: slot 0 = tile w, slot
// 1 = tile w + 4 (all 4 column tiles), slot 2 = tile 8 + w/2 (column tiles
// ctb, ctb + 1).  8 waves: slot 0 = tile w (4 column tiles), no slot 1, slot 2
// = tile 8 + w/4 (column tile ctb = w % 4).  T' of a slot-2 tile belongs to the
// first of the waves sharing it.
template <int NW>
struct Own {
  int ft[3];
  int ctb;
  bool own_t2;
  bool tile8;       // slot 2 is tile 8 (else tile 9)
  int krow0;        // K^T row of the second factor of slot 0: li + w
  __device__ __forceinline__ Own(int w, int li) {
    ft[0] = w;
    ft[1] = w + 4;
    ft[2] = 8 + w / (NW / 2);
    ctb = (w % (NW / 2)) * Waves<NW>::NCT2;
    own_t2 = (w % (NW / 2)) == 0;
    tile8 = ft[2] == 8;
    krow0 = (li + w) & 15;
  }
};

// ---- state images in the workspace (register layout, see above) -----------
// Images and flags move between workgroups that may sit on different XCDs
// (each with its own L2).  Every image access is a buffer access with the
// device-scope cache policy (sc1): stores are written through to where all
// XCDs see them before they count as complete, and loads never hit a stale L2
// line.  So the handover needs no whole-cache write-back or invalidate: the
// writer waits for its stores to complete, then raises the flag (a device-scope
// atomic store); the reader issues its image loads after it has seen the flag.
constexpr int kSC1 = 16;                    // buffer cache policy: device scope
constexpr int kBufWord3 = 0x00020000;       // buffer descriptor word 3 (gfx9: 32-bit data, raw)
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// Loads of the rows of one segment of q, k and v (row r: token t_begin + r of
// sequence bh) through buffer descriptors that span the rows r0 .. r0 + span - 1
// of one call: a row at or past the segment's end reads as zeros (the
// descriptor's range check), which makes the padding of a partial chunk, and a
// chunk past the last one, zero without clamping or masking.  The descriptors
// are rebuilt per call in scalar registers (r0 is wave-uniform), so the offsets
// stay small whatever the sequence length.
struct SegRows {
  const uint16_t *q, *k, *v;
  size_t row0;
  int n;
  __device__ __forceinline__ SegRows(const uint16_t* q_, const uint16_t* k_, const uint16_t* v_, int bh, int N,
                                     int t_begin, int t_end)
      : q(q_), k(k_), v(v_), row0((size_t)bh * N + t_begin), n(t_end - t_begin) {}
  // Lane (li, g) loads row r0 + lr (lr < span): v columns 8g..8g+7 into d[0]
  // and 32+8g..+7 into d[1], and into d[2] dimensions 8g..+7 of k for lanes
  // g < 2, and for lanes g >= 2 dimensions 8(g-2)..+7 of q when WITH_Q, else
  // zeros (an offset past the range: no memory traffic).  The k operand's
  // upper k-slots must hold no k values: a transposing product multiplies
  // them by zero, and 0 * Inf or 0 * NaN would spread a non-finite value
  // across the token's row.
  template <bool WITH_Q>
  __device__ __forceinline__ void load(uint4* d, int r0, int span, int lr, int g) const {
    // (read back from lane 0: the clamps compile to vector instructions, and a
    // descriptor in vector registers would need a loop over distinct values)
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(span, n - r0)));
    const size_t base = row0 + (size_t)__builtin_amdgcn_readfirstlane(max(0, min(r0, n)));
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(v + base * kDV), 0, rows * kDV * 2, kBufWord3);
    d[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, lr * kDV * 2 + 16 * g, 0, 0));
    d[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, lr * kDV * 2 + 64 + 16 * g, 0, 0));
    const int ko = WITH_Q || g < 2 ? lr * kD * 2 + 16 * (g & 1) : 0x40000000;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(k + base * kD), 0, rows * kD * 2, kBufWord3);
    if (WITH_Q && g >= 2) {
      const __amdgpu_buffer_rsrc_t rq =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(q + base * kD), 0, rows * kD * 2, kBufWord3);
      d[2] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, ko, 0, 0));
    } else {
      d[2] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, ko, 0, 0));
    }
  }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t image_rsrc(const float* img) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(img), 0, kImgFloats * 4, kBufWord3);
}

// Writes a (ADD = false) or a + b (ADD = true).
template <int NW, bool ADD>
__device__ __forceinline__ void image_store(float* img, const Acc& a, const Acc& b, int w, int lane) {
  using Sh = Waves<NW>;
  const int li = lane & 15, g = lane >> 4;
  const __amdgpu_buffer_rsrc_t r = image_rsrc(img);
#pragma unroll
  for (int s = 0; s < 3; ++s)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      if (Sh::has(s, ct)) {
        const f32x4 x = ADD ? a.s[s][ct] + b.s[s][ct] : a.s[s][ct];
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r,
                                               ((w * Sh::NCTS + Sh::pair_index(s, ct)) * 64 + lane) * 16, 0, kSC1);
      }
  if (li == 0) {
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const f32x4 x = ADD ? a.t[s] + b.t[s] : a.t[s];
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r,
                                             (kImgS + ((w * 3 + s) * 4 + g) * 4) * 4, 0, kSC1);
    }
  }
}

// This wave's part of the image at img: S' pairs, then T' (lanes li == 0; the
// other lanes read the start of the image and discard it).
template <int NW>
__device__ __forceinline__ void image_load(const float* img, Acc& x, int w, int lane) {
  using Sh = Waves<NW>;
  const int li = lane & 15, g = lane >> 4;
  const __amdgpu_buffer_rsrc_t r = image_rsrc(img);
#pragma unroll
  for (int s = 0; s < 3; ++s)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      if (Sh::has(s, ct))
        x.s[s][ct] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       r, ((w * Sh::NCTS + Sh::pair_index(s, ct)) * 64 + lane) * 16, 0, kSC1));
#pragma unroll
  for (int s = 0; s < 3; ++s)
    x.t[s] = __builtin_bit_cast(
        f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, li == 0 ? (kImgS + ((w * 3 + s) * 4 + g) * 4) * 4 : 0, 0,
                                                     kSC1));
}

template <int NW>
__device__ __forceinline__ void acc_add(Acc& a, const Acc& x, int lane) {
  using Sh = Waves<NW>;
#pragma unroll
  for (int s = 0; s < 3; ++s) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      if (Sh::has(s, ct)) a.s[s][ct] += x.s[s][ct];
    if ((lane & 15) == 0) a.t[s] += x.t[s];
  }
}

// Publish this workgroup's image: every wave waits until its image stores are
// complete, then (after the barrier) one thread raises the flag.
__device__ __forceinline__ void raise_flag(int* flag, int value) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(flag, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait (per wave) until *flag is nonzero and return it; 0 after `limit`
// polls, with the error recorded (the caller then reads whatever the image
// holds: the results are wrong, and the error code says so).
__device__ __forceinline__ int wait_flag(const int* flag, int* err, int limit) {
  for (int i = 0; i < limit; ++i) {
    const int v = __builtin_amdgcn_readfirstlane(__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (v != 0) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      return v;
    }
    __builtin_amdgcn_s_sleep(4);
  }
  __hip_atomic_store(err, kN3ErrTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return 0;
}

// The caller's state is read by every segment of a sequence (for its prefix)
// and overwritten in place by the last one (with the final state).  Every
// segment but the last therefore reports, once its loads of the caller's
// state have completed, on a per-sequence counter (the last segment's flag
// slot, which never carries a flag); the last segment waits for all nseg - 1
// reports before its final store.  The order is the same as for the images:
// every wave waits for its loads to return, the waves meet at a barrier, one
// thread bumps the counter; the writer's stores are issued only after it has
// seen the full count.  The wait is bounded like the others, and nearly free:
// it comes after the last segment's prefix step, which has already waited for
// the group sums that the last readers (the group leaders) publish just before
// they read the caller's state.

__device__ __forceinline__ void report_state_read(int* ctr) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void wait_count(const int* ctr, int want, int* err, int limit) {
  for (int i = 0; i < limit; ++i) {
    const int v = __builtin_amdgcn_readfirstlane(__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (v >= want) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      return;
    }
    __builtin_amdgcn_s_sleep(4);
  }
  __hip_atomic_store(err, kN3ErrTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- the caller's state layout <-> registers ------------------------------
// The [153 x 64] S and [153] T of one head, with the sqrt-multinomial weights
// divided out (load) or applied (store).
constexpr int kAbiImg = kD3 * (kDV + 1);

// The caller's state straight into registers (no LDS, no barrier, so the loads
// can stay in flight during the first pass): raw values first, then the
// sqrt-multinomial weights divided out once they are needed.
template <int NW>
__device__ __forceinline__ void load_caller_state_raw(const float* st_S, const float* st_T, int bh, const Own<NW>& own,
                                                      Acc& a) {
  using Sh = Waves<NW>;
  const int lane = threadIdx.x & 63, li = lane & 15, g = lane >> 4;
  const float* S = st_S + (size_t)bh * kD3 * kDV;
  const float* T = st_T + (size_t)bh * kD3;
  zero_acc(a);
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    if (s == 1 && !Sh::HAS_S1) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float wt;
      const int rc = max(abi_row(own.ft[s], 4 * g + r, &wt), 0);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        a.s[s][ct][r] = Sh::has(s, ct) ? S[rc * kDV + 16 * (s == 2 ? own.ctb + ct : ct) + li] : 0.0f;
      a.t[s][r] = T[rc];
    }
  }
}

template <int NW>
__device__ __forceinline__ void unweight_caller_state(const Own<NW>& own, Acc& a) {
  using Sh = Waves<NW>;
  const int lane = threadIdx.x & 63, li = lane & 15, g = lane >> 4;
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const bool own_t = li == 0 && (s == 0 || (s == 1 && Sh::HAS_S1) || (s == 2 && own.own_t2));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float wt;
      const int row = abi_row(own.ft[s], 4 * g + r, &wt);
      const float sc = 1.0f / wt;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        a.s[s][ct][r] = (row >= 0 && Sh::has(s, ct)) ? a.s[s][ct][r] * sc : 0.0f;
      a.t[s][r] = (row >= 0 && own_t) ? a.t[s][r] * sc : 0.0f;
    }
  }
}

// Stored through LDS as a float image, so that the global stores are full
// 16-byte accesses.
template <int NW>
__device__ __forceinline__ void store_caller_state(float* img, float* st_S, float* st_T, int bh, const Own<NW>& own,
                                                   const Acc& a) {
  using Sh = Waves<NW>;
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  // every row of the image is written by exactly one lane group (zero rows of
  // the internal layout map nowhere)
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    if (s == 1 && !Sh::HAS_S1) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float wt;
      const int row = abi_row(own.ft[s], 4 * g + r, &wt);
      if (row >= 0) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          if (Sh::has(s, ct)) img[row * kDV + 16 * (s == 2 ? own.ctb + ct : ct) + li] = a.s[s][ct][r] * wt;
        if (li == 0 && (s < 2 || own.own_t2)) img[kD3 * kDV + row] = a.t[s][r] * wt;
      }
    }
  }
  __syncthreads();
  float4* ds4 = reinterpret_cast<float4*>(st_S + (size_t)bh * kD3 * kDV);
  float* dt = st_T + (size_t)bh * kD3;
  for (int i = tid; i < kD3 * kDV / 4; i += Sh::NTHREADS)
    __builtin_nontemporal_store(reinterpret_cast<const f32x4*>(img)[i], reinterpret_cast<f32x4*>(ds4) + i);
  for (int i = tid; i < kD3; i += Sh::NTHREADS) __builtin_nontemporal_store(img[kD3 * kDV + i], dt + i);
}

// The final state a + b (the prefix and the segment's own sum) stored straight
// from the accumulators: each wave writes the rows it owns (16 consecutive
// floats of a row per lane group, the T entry from lane li = 0), with no
// barrier and no pass through LDS; every element of S and T is written by
// exactly one lane (zero rows of the internal layout map nowhere).
template <int NW>
__device__ __forceinline__ void store_caller_state_sum(float* st_S, float* st_T, int bh, const Own<NW>& own,
                                                       const Acc& a, const Acc& b) {
  using Sh = Waves<NW>;
  const int lane = threadIdx.x & 63, li = lane & 15, g = lane >> 4;
  float* S = st_S + (size_t)bh * kD3 * kDV;
  float* T = st_T + (size_t)bh * kD3;
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    if (s == 1 && !Sh::HAS_S1) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float wt;
      const int row = abi_row(own.ft[s], 4 * g + r, &wt);
      if (row >= 0) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          if (Sh::has(s, ct))
            __builtin_nontemporal_store((a.s[s][ct][r] + b.s[s][ct][r]) * wt,
                                        &S[row * kDV + 16 * (s == 2 ? own.ctb + ct : ct) + li]);
        if (li == 0 && (s < 2 || own.own_t2)) __builtin_nontemporal_store((a.t[s][r] + b.t[s][r]) * wt, &T[row]);
      }
    }
  }
}

// ---- the replay: one pass over the chunks [t_begin, t_end) of sequence bh ---
// from the state a: the outputs of every token, and a += the segment's sum.
template <int C, int NW_, typename TOUT>
__device__ __forceinline__ void segment_pass(Lds<C>& L, const Own<NW_>& own, Acc& a, const uint16_t* __restrict__ q,
                                             const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                             TOUT* __restrict__ o, int bh, int N, int t_begin, int t_end,
                                             float inv_a, bool keep_state) {
  using Sh = Shape<C, NW_>;
  constexpr int NKB = Sh::NKB, NW = Sh::NW, NCT2 = Sh::NCT2;
  constexpr bool HAS_S1 = Sh::HAS_S1;
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nchunks = (t_end - t_begin + C - 1) / C;
  if (nchunks <= 0) return;  // uniform
  f32x4(&acc)[3][4] = a.s;
  f32x4(&tacc)[3] = a.t;
  const int ctb = own.ctb;
  const bool own_t2 = own.own_t2;

  // ---- global loads.  Wave w loads its own token tile 16w .. 16w + 15:
  //      lane (li, g) takes columns 8g..8g+7 and 32+8g..+7 of v for token li of
  //      the tile, and k (g < 2) or q (g >= 2) dimensions 8(g%2)..+7: the
  //      natural row-major 16-byte pieces, which are exactly the A operand of
  //      the transposing MFMAs in `stage`.  Chunk c is loaded into register set
  //      c % DEPTH, DEPTH chunks ahead of its use.  The loads are buffer loads
  //      over the segment's rows: a token past the segment's end (the padding
  //      of a partial chunk, or a chunk past the last) reads zeros, so padding
  //      tokens need no clamping or masking, and every load is issued
  //      unconditionally, so the waits for them are exact.
  constexpr int TPW = Sh::TPW;
  constexpr int NPF = 3 * TPW;
  constexpr int DEPTH = 2;  // register sets of prefetched loads
  uint4 pf[DEPTH][NPF];
  const SegRows rows(q, k, v, bh, N, t_begin, t_end);
  auto issue_loads = [&](uint4 (&pfs)[NPF], int chunk) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) rows.load<true>(pfs + 3 * i, chunk * C, C, 16 * (w + NW * i) + li, g);
  };
  // One-hot B operands: sel0 picks k-slots 0..15 and sel1 k-slots 16..31 of a
  // 16x16x32 product, so that A . sel = the A rows transposed into the
  // accumulator layout (lane (n, g) then holds rows 4g..4g+3 of column n).
  // Exact: every product is a bfloat16 value times 1 or 0.
  bf16x8 sel0, sel1;
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
  // (padding tokens arrive as zeros; the q pieces of lanes g >= 2 are zeroed
  // in the k operand: sel0 multiplies its k-slots 16..31 by zero, which would
  // turn a non-finite q value into a NaN row of K^T)
  auto stage = [&](const uint4 (&pfs)[NPF], int b) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tt = w + NW * i;
      const bf16x8 v0 = __builtin_bit_cast(bf16x8, pfs[3 * i]);
      const bf16x8 v1 = __builtin_bit_cast(bf16x8, pfs[3 * i + 1]);
      const bf16x8 ka = __builtin_bit_cast(bf16x8, g < 2 ? pfs[3 * i + 2] : make_uint4(0, 0, 0, 0));
      // V^T: four 16x16 tiles, lane (li, g) gets tokens 16tt + 4g + r of column 16ct + li
      const f32x4 d0 = mfma_bf16_k32(v0, sel0, zero);
      const f32x4 d1 = mfma_bf16_k32(v0, sel1, zero);
      const f32x4 d2 = mfma_bf16_k32(v1, sel0, zero);
      const f32x4 d3 = mfma_bf16_k32(v1, sel1, zero);
      const f32x4 dv[4] = {d0, d1, d2, d3};
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int c = 16 * ct + li;
        *reinterpret_cast<uint2*>(&L.V[b][c][swz(c, 16 * tt + 4 * g)]) =
            make_uint2(pack2(dv[ct][0], dv[ct][1]), pack2(dv[ct][2], dv[ct][3]));
      }
      // K^T (float): lane (li, g) gets dimension li of tokens 16tt + 4g + r
      const f32x4 dk = mfma_bf16_k32(ka, sel0, zero);
      *reinterpret_cast<f32x4*>(&L.K[b][li][16 * tt + 4 * g]) = dk;
      if (g >= 2) {
        // q / a, rounded to bfloat16 (exact for a = 1): then q.k comes out
        // already divided by a, and the query features need no scaling
        const uint4 raw = pfs[3 * i + 2];
        const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
        uint32_t sc[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[e] = pack2(lo_f(wd[e]) * inv_a, hi_f(wd[e]) * inv_a);
        uint16_t* d = &L.Q[b][16 * tt + li][8 * (g - 2)];
        *reinterpret_cast<uint2*>(d) = make_uint2(sc[0], sc[1]);
        *reinterpret_cast<uint2*>(d + 4) = make_uint2(sc[2], sc[3]);
        *reinterpret_cast<uint2*>(d + 16) = make_uint2(sc[0], sc[1]);
        *reinterpret_cast<uint2*>(d + 20) = make_uint2(sc[2], sc[3]);
      }
    }
  };
  // bfloat16 copy of the state (k-slot order) and T for the next state read
  auto publish = [&](int b) {
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      if (s == 1 && !HAS_S1) continue;
      const int ks = kslot_of(own.ft[s], 4 * g);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        if (Sh::has(s, ct)) {
          const int c = 16 * (s == 2 ? ctb + ct : ct) + li;
          *reinterpret_cast<uint2*>(&L.S[b][c][ks]) =
              make_uint2(pack2(acc[s][ct][0], acc[s][ct][1]), pack2(acc[s][ct][2], acc[s][ct][3]));
        }
      }
      if (li == 0 && (s < 2 || own_t2)) {
        float hi[4], lo[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          hi[r] = (float)f32_to_bf16(tacc[s][r]);
          lo[r] = tacc[s][r] - hi[r];
        }
        *reinterpret_cast<uint2*>(&L.T[b][0][ks]) = make_uint2(pack2(hi[0], hi[1]), pack2(hi[2], hi[3]));
        *reinterpret_cast<uint2*>(&L.T[b][1][ks]) = make_uint2(pack2(lo[0], lo[1]), pack2(lo[2], lo[3]));
      }
    }
  };

  // chunk c lives in register set c % DEPTH; chunks 1..DEPTH are in flight
  // when the loop starts, and body(j) refills the set it stages from with
  // chunk j + 1 + DEPTH
  issue_loads(pf[0], 0);
  stage(pf[0], 0);
#pragma unroll
  for (int c = 1; c <= DEPTH; ++c) issue_loads(pf[c % DEPTH], c);
  publish(0);
  __syncthreads();

  const int h = g & 1, gh = g >> 1;

  // Outputs of the chunk computed last, stored at the start of the next
  // iteration (after that iteration's inputs are staged), so that the wait for
  // the staged loads never waits for fresh stores.
  f32x4 yo[TPW][5];
  int prev_t0 = -1, prev_nv = 0;
  auto store_prev = [&]() {
    if (prev_t0 >= 0) {  // uniform
#pragma unroll
      for (int tw = 0; tw < TPW; ++tw) {
        // o = Y[:d_v] / Y[d_v]: the normaliser of token li sits in rows 0 and 1
        // of column tile 4 (lanes 0..15); every lane takes part in the shuffle
        const float inv = __builtin_amdgcn_rcpf(__shfl(yo[tw][4][0] + yo[tw][4][1], li));  // within 1 ulp
        const int tok = 16 * (w + NW * tw) + li;
        if (tok < prev_nv) {
          TOUT* orow = o + ((size_t)bh * N + prev_t0 + tok) * kDV + 4 * g;
          // non-temporal: the outputs are not read again by this kernel
          if constexpr (std::is_same_v<TOUT, float>) {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
              __builtin_nontemporal_store(yo[tw][ct] * inv, reinterpret_cast<f32x4*>(orow + 16 * ct));
          } else {
            typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
              __builtin_nontemporal_store(u32x2{pack2(yo[tw][ct][0] * inv, yo[tw][ct][1] * inv),
                                                pack2(yo[tw][ct][2] * inv, yo[tw][ct][3] * inv)},
                                          reinterpret_cast<u32x2*>(orow + 16 * ct));
          }
        }
      }
    }
  };

  auto body = [&](int j, uint4 (&pfs)[NPF]) {
    const int b = j & 1;
    const int t0 = t_begin + j * C;
    const int nv = min(C, t_end - t0);
    if (j + 1 < nchunks) stage(pfs, b ^ 1);
    issue_loads(pfs, j + 1 + DEPTH);
    store_prev();

    // The update comes first: the state read below only uses the previous
    // chunk's copy of the state, and by the time this chunk's copy is
    // published the update's products have long completed.
    // ---- state update: S' += phi(K)^T V on the owned feature tiles, T' += phi(K)^T 1
    //      Lane li holds row li of K^T (x_li) and row li + w (the second factor
    //      of tile w); the second factors of the other tiles are those rows as
    //      held by other lanes of the same 16-lane row (DPP rotations), so only
    //      two rows come from LDS.  Padding tokens have k = 0 and v = 0, so
    //      every product with x, and every product with v, vanishes for them;
    //      the constant feature is 1 for every token of the chunk, and its T'
    //      entry is corrected by the number of padding tokens.
    //      The last chunk's update only matters for the final state (keep_state).
    if (j + 1 < nchunks || keep_state) {  // uniform
      const uint32_t one2 = li == 0 ? 0x3F803F80u : 0u;
      const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(one2, one2, one2, one2));
      const bf16x8 zeros = __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u));
      const float pair_m = li < 8 ? 1.0f : 0.0f, const_m = li == 8 ? 1.0f : 0.0f;  // rows of tile 8
      const bool tile8 = own.tile8;  // wave-uniform
      // The update and the state read run at raised wave priority: with two
      // waves per SIMD, the wave in a run of matrix products issues first and
      // the other wave's vector work fills the gaps.
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int t8 = 32 * kb + 8 * g;
        float xi[8], xa[8];
        {
          const float4 a0 = *reinterpret_cast<const float4*>(&L.K[b][li][t8]);
          const float4 a1 = *reinterpret_cast<const float4*>(&L.K[b][li][t8 + 4]);
          xi[0] = a0.x; xi[1] = a0.y; xi[2] = a0.z; xi[3] = a0.w;
          xi[4] = a1.x; xi[5] = a1.y; xi[6] = a1.z; xi[7] = a1.w;
          const float4 c0 = *reinterpret_cast<const float4*>(&L.K[b][own.krow0][t8]);
          const float4 c1 = *reinterpret_cast<const float4*>(&L.K[b][own.krow0][t8 + 4]);
          xa[0] = c0.x; xa[1] = c0.y; xa[2] = c0.z; xa[3] = c0.w;
          xa[4] = c1.x; xa[5] = c1.y; xa[6] = c1.z; xa[7] = c1.w;
        }
        bf16x8 vb[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const int c = 16 * ct + li;
          vb[ct] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&L.V[b][c][swz(c, t8)]));
        }
#pragma unroll
        for (int s = 0; s < 3; ++s) {
          if (s == 1 && !HAS_S1) continue;
          float f[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (s == 0) {
              f[e] = xi[e] * xa[e];                       // tile w: x_li x_(li+w)
            } else if (s == 1) {
              f[e] = xi[e] * from_lane_plus<4>(xa[e]);    // tile w + 4: x_li x_(li+w+4)
            } else {
              f[e] = xi[e];  // tile 9: x_li (tile 8 below)
            }
          }
          // tile 8: x_li x_(li+8) (li < 8), the constant (li == 8), zero rows.
          // The branch is wave-uniform, so every lane runs the DPP rotation,
          // which reads its source from the other lanes of the row.
          if (s == 2 && tile8) {
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = fmaf(xi[e] * from_lane_plus<8>(xi[e]), pair_m, const_m);
          }
          const bf16x8 aphi = __builtin_bit_cast(
              bf16x8, make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])));
          if (s < 2) {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) acc[s][ct] = mfma_bf16_k32(aphi, vb[ct], acc[s][ct]);
            tacc[s] = mfma_bf16_k32(aphi, ones, tacc[s]);
          } else {
            // (every wave runs the T product, against zeros where it does not
            // own T of the tile: no branch in the loop)
            tacc[2] = mfma_bf16_k32(aphi, own_t2 ? ones : zeros, tacc[2]);
            // column tiles ctb .. ctb + NCT2 - 1 (ctb is wave-uniform; operands
            // selected, not branched on)
            if constexpr (NCT2 == 2) {
              acc[2][0] = mfma_bf16_k32(aphi, ctb == 0 ? vb[0] : vb[2], acc[2][0]);
              acc[2][1] = mfma_bf16_k32(aphi, ctb == 0 ? vb[1] : vb[3], acc[2][1]);
            } else {
              acc[2][0] = mfma_bf16_k32(aphi, ctb == 0 ? vb[0] : ctb == 1 ? vb[1] : ctb == 2 ? vb[2] : vb[3],
                                        acc[2][0]);
            }
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }

#pragma unroll
    for (int tw = 0; tw < TPW; ++tw) {
      const int tt = w + NW * tw;  // token tile, wave-uniform
      const int tok = 16 * tt + li;

      // ---- diagonal block: P = tril(p_3(K Q^T / a)), lane holds P[token li][keys]
      const bf16x4 bq = __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(&L.Q[b][tok][4 * g]));
      // Scores of every key tile first (straight-line: the key reads and the
      // products of different tiles overlap), then the polynomial only for
      // the key tiles up to the token tile (wave-uniform branches); later
      // tiles are zero, and only the diagonal tile is masked causally (key
      // 16 kt + 4g + r against token 16 tt + li).
      f32x4 sc[2 * NKB];
#pragma unroll
      for (int kt = 0; kt < 2 * NKB; ++kt) {
        const int key0 = 16 * kt + li;
        const uint2 ak = make_uint2(pack2(L.K[b][4 * g][key0], L.K[b][4 * g + 1][key0]),
                                    pack2(L.K[b][4 * g + 2][key0], L.K[b][4 * g + 3][key0]));
        sc[kt] = mfma_bf16_k16(__builtin_bit_cast(bf16x4, ak), bq, f32x4{0.f, 0.f, 0.f, 0.f});
      }
      bf16x8 pb[NKB];
#pragma unroll
      for (int kt = 0; kt < 2 * NKB; ++kt) {
        float p[4] = {0.f, 0.f, 0.f, 0.f};
        if (kt <= tt) {
#pragma unroll
          for (int r = 0; r < 4; ++r) p[r] = fmaf(sc[kt][r], fmaf(0.5f, sc[kt][r], 1.0f), 1.0f);  // s = q.k / a
          if (kt == tt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] = 4 * g + r <= li ? p[r] : 0.0f;
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) pb[kt >> 1][4 * (kt & 1) + r] = f32_to_bf16(p[r]);
      }

      f32x4 y[5];
#pragma unroll
      for (int ct = 0; ct < 5; ++ct) y[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      // Y^T += [V, 1]^T P^T; row l of column tile ct is value column 16 ct + l, so
      // lane (li, g) ends up with columns 16 ct + 4g .. 16 ct + 4g + 3 of token li
      const uint32_t one2 = li == 0 ? 0x3F803F80u : 0u;
      const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(one2, one2, one2, one2));
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if (2 * kb <= tt) {
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            const int c = 16 * ct + li;
            const uint2 v0 = *reinterpret_cast<const uint2*>(&L.V[b][c][swz(c, 32 * kb + 4 * g)]);
            const uint2 v1 = *reinterpret_cast<const uint2*>(&L.V[b][c][swz(c, 32 * kb + 16 + 4 * g)]);
            y[ct] = mfma_bf16_k32(__builtin_bit_cast(bf16x8, make_uint4(v0.x, v0.y, v1.x, v1.y)), pb[kb], y[ct]);
          }
          y[4] = mfma_bf16_k32(ones, pb[kb], y[4]);
        }
      }

      // ---- state read: Y^T += S'^T phi'(q)^T, features built in registers
      float yv[16], zv[16];
      {
        const uint16_t* qrow = &L.Q[b][tok][0];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint2 t2 = *reinterpret_cast<const uint2*>(qrow + 8 * h + 4 * e);
          yv[4 * e] = lo_f(t2.x); yv[4 * e + 1] = hi_f(t2.x);
          yv[4 * e + 2] = lo_f(t2.y); yv[4 * e + 3] = hi_f(t2.y);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t t1 = *reinterpret_cast<const uint32_t*>(qrow + 8 * h + 2 * gh + 2 * e);
          zv[2 * e] = lo_f(t1);
          zv[2 * e + 1] = hi_f(t1);
        }
      }
      // q is staged as q / a: the products y_s z_t already carry 2 alpha_2 = 1 / a^2,
      // y_s carries alpha_1 = 1 / a
      const float kb0f = gh == 0 ? 0.5f : 1.0f;  // diagonal tile: weight 1 instead of 2
      const float cB = g >= 2 ? 1.0f : 0.0f, cC = g == 1 ? 1.0f : 0.0f;
      constexpr int kD0[4] = {0, 1, 4, 5};
      __builtin_amdgcn_s_setprio(1);
      // (a scheduling hint that interleaves the state copy's LDS reads with the
      // products: about 0.5 us per call)
      __builtin_amdgcn_iglp_opt(1);
#pragma unroll
      for (int kb = 0; kb < 5; ++kb) {
        float f[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          if (kb < 4) {
            f[s] = yv[s] * zv[(s + kD0[kb]) & 15];
            if (kb == 0) f[s] *= kb0f;
          } else {
            // lane groups: 0 pairs at distance 8, 1 the constant (k-slot 0),
            // 2 and 3 linear: one select and one product per feature
            const float m = g == 0 ? zv[(s + 8) & 15] : cB;
            f[s] = s == 0 ? fmaf(yv[s], m, cC) : yv[s] * m;
          }
        }
        const bf16x8 bphi = __builtin_bit_cast(
            bf16x8, make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])));
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const uint4 a4 = *reinterpret_cast<const uint4*>(&L.S[b][16 * ct + li][32 * kb + 8 * g]);
          y[ct] = mfma_bf16_k32(__builtin_bit_cast(bf16x8, a4), bphi, y[ct]);
        }
        // normaliser: rows 0 / 1 of column tile 4 are T' (high / low bfloat16
        // parts); rows 2..15 repeat them and are never read (so every lane
        // reads one of two words per lane group: a broadcast)
        const uint4 tA = *reinterpret_cast<const uint4*>(&L.T[b][li & 1][32 * kb + 8 * g]);
        y[4] = mfma_bf16_k32(__builtin_bit_cast(bf16x8, tA), bphi, y[4]);
      }
      __builtin_amdgcn_s_setprio(0);

      // ---- epilogue (normalised and stored at the start of the next iteration,
      //      when the products have long completed)
#pragma unroll
      for (int ct = 0; ct < 5; ++ct) yo[tw][ct] = y[ct];
    }
    prev_t0 = t0;
    prev_nv = nv;

    // the constant feature counted the padding tokens of a partial chunk:
    // take them out of its T' entry (row 8 of tile 8: lane 32, element 0)
    tacc[2][0] -= (own.tile8 && own_t2 && lane == 32) ? (float)(C - nv) : 0.0f;

    if (j + 1 < nchunks) publish(b ^ 1);
    __syncthreads();
  };
  for (int j0 = 0; j0 < nchunks; j0 += DEPTH) {
#pragma unroll
    for (int i = 0; i < DEPTH; ++i)
      if (j0 + i < nchunks) body(j0 + i, pf[(i + 1) % DEPTH]);
  }
  store_prev();
}

// ---- segment sum in registers ---------------------------------------------
// A = sum over the segment of phi(k)^T [v, 1], without staging anything in LDS:
// every wave takes whole 32-token groups (wave w: groups w, w + NW, ...) and
// keeps a full partial state in registers: 10 feature tiles x 4 column tiles
// of accumulators, and T of tile f in column f of one more tile (B operand:
// ones in column f).  It loads the group's k and v once, transposes them on
// the matrix cores (one-hot selector products, as in segment_pass) straight
// into operand registers and builds the features with DPP rotations.  At the
// end the partial states are added up in LDS, one wave's state at a time (a
// fixed order, so the result does not depend on timing), and every wave picks
// up the tiles it owns in the replay.
// bytes of the reduction area: one state of 41 tiles
template <int NW>
constexpr int sum_lds_bytes() { return 41 * 64 * 16; }

template <int NW>
__device__ __forceinline__ void segment_sum_regs(unsigned char* lds_raw, const Own<NW>& own, Acc& a,
                                                 const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                 int bh, int N, int t_begin, int t_end) {
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ngroups = (t_end - t_begin + 31) / 32;

  f32x4 F[10][4], Tp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int f = 0; f < 10; ++f)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) F[f][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  // loads of group G: per 16-token tile, v columns 8g..+7 and 32+8g..+7 and
  // (lanes g < 2) k dimensions 8g..+7 of token li; tokens past the segment's
  // end (and a group past the last) read as zeros
  const SegRows rows(nullptr, k, v, bh, N, t_begin, t_end);
  auto issue = [&](uint4 (&r)[6], int G) {
#pragma unroll
    for (int x = 0; x < 2; ++x) rows.load<false>(r + 3 * x, 32 * G, 32, 16 * x + li, g);
  };
  bf16x8 sel0, sel1;
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
  const float pair_m = li < 8 ? 1.0f : 0.0f, const_m = li == 8 ? 1.0f : 0.0f;  // rows of tile 8
  int pad = 0;  // padding tokens seen (their constant feature is 1)

  // group G from the loaded registers r; `refill` is called once r has been
  // consumed (it issues the loads of the next group into r)
  auto group = [&](uint4 (&r)[6], int G, auto&& refill) {
    const int nvalid = min(32, t_end - (t_begin + 32 * G));
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    uint32_t vw[4][4];  // B operands of the 4 column tiles, built in place
    float xi[8];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      // (padding tokens arrive as zeros, and so do k-slots 16..31 of the k
      // operand: lanes g >= 2 load nothing there)
      const bf16x8 v0 = __builtin_bit_cast(bf16x8, r[3 * x]);
      const bf16x8 v1 = __builtin_bit_cast(bf16x8, r[3 * x + 1]);
      const bf16x8 ka = __builtin_bit_cast(bf16x8, r[3 * x + 2]);
      const f32x4 d0 = mfma_bf16_k32(v0, sel0, zero), d1 = mfma_bf16_k32(v0, sel1, zero);
      const f32x4 d2 = mfma_bf16_k32(v1, sel0, zero), d3 = mfma_bf16_k32(v1, sel1, zero);
      const f32x4 dv[4] = {d0, d1, d2, d3};
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        vw[ct][2 * x] = pack2(dv[ct][0], dv[ct][1]);
        vw[ct][2 * x + 1] = pack2(dv[ct][2], dv[ct][3]);
      }
      // lane (li, g): dimension li of tokens 16x + 4g .. 16x + 4g + 3
      const f32x4 dk = mfma_bf16_k32(ka, sel0, zero);
#pragma unroll
      for (int e = 0; e < 4; ++e) xi[4 * x + e] = dk[e];
    }
    refill();
    // k-slots of lane group g: tokens 4g..4g+3 and 16+4g..16+4g+3 of the group
    bf16x8 vb[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) vb[ct] = __builtin_bit_cast(bf16x8, make_uint4(vw[ct][0], vw[ct][1], vw[ct][2], vw[ct][3]));
    // features of tile f (compile-time: the DPP rotation is an immediate)
    auto tile = [&](auto fc) {
      constexpr int f = decltype(fc)::value;
      float fx[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (f == 0) fx[e] = xi[e] * xi[e];                        // x_li^2
        else if constexpr (f < 8) fx[e] = xi[e] * from_lane_plus<f>(xi[e]);  // x_li x_(li+f)
        else if constexpr (f == 8) fx[e] = fmaf(xi[e] * from_lane_plus<8>(xi[e]), pair_m, const_m);
        else fx[e] = xi[e];                                                   // linear
      }
      const bf16x8 aphi = __builtin_bit_cast(
          bf16x8, make_uint4(pack2(fx[0], fx[1]), pack2(fx[2], fx[3]), pack2(fx[4], fx[5]), pack2(fx[6], fx[7])));
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) F[f][ct] = mfma_bf16_k32(aphi, vb[ct], F[f][ct]);
      // ones in column f of the T tile (rebuilt here on purpose: ten such
      // operands kept across the loop would not fit in registers)
      uint32_t one2 = li == f ? 0x3F803F80u : 0u;
      asm volatile("" : "+v"(one2));
      Tp = mfma_bf16_k32(aphi, __builtin_bit_cast(bf16x8, make_uint4(one2, one2, one2, one2)), Tp);
    };
    tile(std::integral_constant<int, 0>{});
    tile(std::integral_constant<int, 1>{});
    tile(std::integral_constant<int, 2>{});
    tile(std::integral_constant<int, 3>{});
    tile(std::integral_constant<int, 4>{});
    tile(std::integral_constant<int, 5>{});
    tile(std::integral_constant<int, 6>{});
    tile(std::integral_constant<int, 7>{});
    tile(std::integral_constant<int, 8>{});
    tile(std::integral_constant<int, 9>{});
    pad += 32 - nvalid;
  };

  // the next group's loads are in flight while this group's products run
  uint4 ra[6];
  issue(ra, w);
  for (int G = w; G < ngroups; G += NW) group(ra, G, [&] { issue(ra, G + NW); });
  // the constant feature counted padding tokens: take them out of its T entry
  // (column 8 = tile 8, row 8: lane 40, element 0)
  Tp[0] -= (lane == 40) ? (float)pad : 0.0f;

  // ---- add up the waves' partial states in LDS, then hand every wave the
  //      tiles it owns.  The 41 tiles form NW parts (part of tile t:
  //      t * NW / 41); in round r wave w adds its partial of part
  //      (w + r) mod NW (round 0 stores it), so every round keeps all waves
  //      busy on different parts and each part is summed in a fixed order
  //      (waves p, p - 1, ..., p - NW + 1 mod NW).
  static_assert((NW & (NW - 1)) == 0, "NW is a power of two");
  f32x4* R = reinterpret_cast<f32x4*>(lds_raw);  // [41 tiles][64 lanes]
  auto at = [&](int t) { return R + t * 64 + lane; };
  auto part = [](int t) { return t * NW / 41; };
  __syncthreads();  // the LDS area may still be in use by earlier code
#pragma unroll
  for (int r = 0; r < NW; ++r) {
    const int pr = (w + r) & (NW - 1);  // uniform
    if (r > 0) __syncthreads();
#pragma unroll
    for (int f = 0; f < 10; ++f)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        if (part(4 * f + ct) == pr) {
          if (r == 0) *at(4 * f + ct) = F[f][ct];
          else *at(4 * f + ct) += F[f][ct];
        }
    if (part(40) == pr) {
      if (r == 0) *at(40) = Tp;
      else *at(40) += Tp;
    }
  }
  __syncthreads();
  using Wv = Waves<NW>;
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    if (s == 1 && !Wv::HAS_S1) {
      a.t[s] = f32x4{0.f, 0.f, 0.f, 0.f};
      continue;
    }
    const int ft = own.ft[s];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      if (Wv::has(s, ct)) a.s[s][ct] = *at(4 * ft + (s == 2 ? own.ctb + ct : ct));
    // T of tile ft: column ft of the T tile, i.e. lane (li = ft, g) of it
    const f32x4 tcol = R[40 * 64 + 16 * g + ft];
    const bool own_t = li == 0 && (s < 2 || own.own_t2);
    a.t[s] = own_t ? tcol : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();  // the area is reused by the replay's buffers
}

// ---- the kernel -------------------------------------------------------------
// Grid: BH * nseg workgroups.  sync == nullptr exactly when nseg == 1 (then
// workgroup b runs sequence b from the caller's state, with no prefix step).
template <int C>
constexpr int waves_for() { return C == 128 ? 8 : 4; }

template <int C, typename TOUT>
__global__ __launch_bounds__(64 * waves_for<C>(), (C == 64 ? 2 : 1)) void prefill_n3_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    TOUT* __restrict__ o, float* __restrict__ st_S, float* __restrict__ st_T, int* __restrict__ sync,
    float* __restrict__ sums, int N, int nseg, int cps, int gs, float inv_a, int wait_limit) {
  constexpr int NW = waves_for<C>();
  using LB = Lds<C>;
  // The replay's chunk buffers, the sum pass's reduction area, and while the
  // final state of a single segment is stored, a float [153 * 65] image of it
  // in the caller's layout.
  constexpr size_t kA = sizeof(LB) > (size_t)sum_lds_bytes<NW>() ? sizeof(LB) : (size_t)sum_lds_bytes<NW>();
  constexpr size_t kLdsBytes = kA > kAbiImg * 4 ? kA : kAbiImg * 4;
  __shared__ __align__(16) unsigned char lds_raw[kLdsBytes];
  __shared__ int s_ticket;
  float* img = reinterpret_cast<float*>(lds_raw);

  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15;
  // wave index in a scalar register: every branch around an MFMA is uniform
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  int ticket = blockIdx.x;
  if (sync != nullptr) {  // uniform
    // the sequence (XCD-affine); its counter gives the segment
    const int b = sequence_of_workgroup(blockIdx.x, nseg, gridDim.x / nseg);
    if (tid == 0)
      s_ticket = b * nseg + __hip_atomic_fetch_add(&sync[kHdr + (size_t)b * nseg * kFlagStride + kTicketWord], 1,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    ticket = __builtin_amdgcn_readfirstlane(s_ticket);
  }
  const int bh = ticket / nseg, seg = ticket % nseg;
  const int t_begin = seg * cps * C;
  const int t_end = min(N, t_begin + cps * C);
  const Own<NW> own(w, li);
  const size_t head0 = (size_t)bh * nseg;  // slot of segment 0 of this sequence
  auto flag_of = [&](int j) { return &sync[kHdr + (head0 + j) * kFlagStride]; };
  auto image_of = [&](int j) { return sums + (head0 + j) * kImgFloats; };
  const int grp = seg / gs, g0 = grp * gs;
  // the last member of a group publishes the group's sum, unless no group follows
  const bool leader = seg == g0 + gs - 1 && seg < nseg - 1;

  // 1. the segment's own sum (that of the last of several segments is part of
  //    the final state; a single segment carries its state through the replay)
  Acc acc;
  if (nseg > 1) segment_sum_regs<NW>(lds_raw, own, acc, k, v, bh, N, t_begin, t_end);
  else zero_acc(acc);
  // a segment that is not the last of its group publishes its sum at once
  if (nseg > 1 && !leader && seg < nseg - 1) {  // uniform
    image_store<NW, false>(image_of(seg), acc, acc, w, lane);
    raise_flag(flag_of(seg), 1);
  }
  // Every segment's prefix starts from the caller's state, loaded after the
  // publication (which waits for all outstanding memory operations); a leader
  // loads it only after it has published the group sum.
  Acc pre;
  if (leader) {
    zero_acc(pre);
  } else {
    load_caller_state_raw<NW>(st_S, st_T, bh, own, pre);
    unweight_caller_state<NW>(own, pre);
    if (nseg > 1 && seg < nseg - 1) report_state_read(flag_of(nseg - 1));  // uniform
  }
  // 2. prefix = caller's state + sums of the earlier members of the group +
  //    group sums of the earlier groups (the leader adds the members' sums to
  //    its own as well, and publishes that as the group sum)
  if (nseg > 1) {  // uniform
    int* err = &sync[1];
    const int r = seg - g0;  // earlier members
    auto source = [&](int i) { return i < r ? g0 + i : (i - r) * gs + gs - 1; };
    if (leader) {
      for (int j = g0; j < seg; j += 2) {
        const bool two = j + 1 < seg;  // uniform
        Acc x, y;
        wait_flag(flag_of(j), err, wait_limit);
        if (two) wait_flag(flag_of(j + 1), err, wait_limit);
        image_load<NW>(image_of(j), x, w, lane);
        image_load<NW>(image_of(two ? j + 1 : j), y, w, lane);
        acc_add<NW>(pre, x, lane);
        acc_add<NW>(acc, x, lane);
        if (two) {
          acc_add<NW>(pre, y, lane);
          acc_add<NW>(acc, y, lane);
        }
      }
      image_store<NW, false>(image_of(seg), acc, acc, w, lane);
      raise_flag(flag_of(seg), 1);
      Acc x;
      load_caller_state_raw<NW>(st_S, st_T, bh, own, x);
      unweight_caller_state<NW>(own, x);
      report_state_read(flag_of(nseg - 1));
      acc_add<NW>(pre, x, lane);
      for (int G = 0; G < grp; ++G) {
        wait_flag(flag_of(G * gs + gs - 1), err, wait_limit);
        image_load<NW>(image_of(G * gs + gs - 1), x, w, lane);
        acc_add<NW>(pre, x, lane);
      }
    } else {
      // two images in flight at a time
      const int n = r + grp;
      for (int i = 0; i < n; i += 2) {
        const bool two = i + 1 < n;  // uniform
        Acc x, y;
        wait_flag(flag_of(source(i)), err, wait_limit);
        if (two) wait_flag(flag_of(source(i + 1)), err, wait_limit);
        image_load<NW>(image_of(source(i)), x, w, lane);
        image_load<NW>(image_of(two ? source(i + 1) : source(i)), y, w, lane);
        acc_add<NW>(pre, x, lane);
        if (two) acc_add<NW>(pre, y, lane);
      }
    }
  }
  // the last of several segments has the final state = its prefix + its own
  // sum now, and stores it before its replay (once every other segment has
  // read the caller's state), so that the store is off the kernel's tail
  if (nseg > 1 && seg == nseg - 1) {  // uniform
    wait_count(flag_of(nseg - 1), nseg - 1, &sync[1], wait_limit);
    store_caller_state_sum<NW>(st_S, st_T, bh, own, pre, acc);
  }
  // 3. replay from the prefix (a single segment also carries the state to the end)
  segment_pass<C, NW, TOUT>(*reinterpret_cast<LB*>(lds_raw), own, pre, q, k, v, o, bh, N, t_begin, t_end, inv_a,
                            nseg == 1);
  if (nseg == 1) store_caller_state<NW>(img, st_S, st_T, bh, own, pre);  // uniform
}

// Clears the error code and the nslots flag slots (flag and ticket words), and
// marks the header as this kernel's.
static __global__ void clear_flags_kernel(int* sync, int nslots) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nslots) {
    sync[kHdr + (size_t)i * kFlagStride] = 0;
    sync[kHdr + (size_t)i * kFlagStride + kTicketWord] = 0;
  }
  if (i < 3) sync[i] = i == 2 ? kN3Magic : 0;
}

// Segments per group: about sqrt(nseg), at least 2.
inline int group_size(int nseg) {
  int gs = 2;
  while (gs * gs < nseg) ++gs;
  return gs;
}

template <int C, typename TOUT>
hipError_t launch(const PrefillArgs& a) {
  const PrefillPlan& pl = a.plan;
  float* st_S = a.state;
  float* st_T = a.state + (size_t)a.BH * kD3 * kDV;
  const float inv_a = 1.0f / a.a;
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* k = static_cast<const uint16_t*>(a.k);
  const uint16_t* v = static_cast<const uint16_t*>(a.v);
  hipEvent_t* ev = a.events;
  int* sync = nullptr;
  float* sums = nullptr;
  if (ev) (void)hipEventRecord(ev[0], a.stream);
  if (pl.nseg > 1) {
    const size_t hdr = header_words(a.BH, pl.nseg);
    sync = reinterpret_cast<int*>(a.workspace);
    sums = a.workspace + hdr;
    const int nslots = a.BH * pl.nseg;
    hipLaunchKernelGGL(clear_flags_kernel, dim3((nslots + 255) / 256), dim3(256), 0, a.stream, sync, nslots);
  }
  if (ev) {
    // events 2 and 3 are recorded by the dispatch itself, at the kernel's
    // start and end (no launch gap inside the interval)
    (void)hipEventRecord(ev[1], a.stream);
    hipExtLaunchKernelGGL((prefill_n3_kernel<C, TOUT>), dim3(a.BH * pl.nseg), dim3(64 * waves_for<C>()), 0, a.stream,
                          ev[2], ev[3], 0, q, k, v, static_cast<TOUT*>(a.o), st_S, st_T, sync, sums, a.N, pl.nseg,
                          pl.chunks_per_seg, group_size(pl.nseg), inv_a, a.wait_limit);
  } else {
    hipLaunchKernelGGL((prefill_n3_kernel<C, TOUT>), dim3(a.BH * pl.nseg), dim3(64 * waves_for<C>()), 0, a.stream,
                       q, k, v, static_cast<TOUT*>(a.o), st_S, st_T, sync, sums, a.N, pl.nseg, pl.chunks_per_seg,
                       group_size(pl.nseg), inv_a, a.wait_limit);
  }
  return hipGetLastError();
}

}  // namespace n3

#ifdef TAYLOR_N3_C128_UNIT
// The 128-token instances live in their own translation unit.  Both units are
// compiled with the instruction scheduler that maximises instruction-level
// parallelism, which measured faster than the default one for each of them.
hipError_t launch_prefill_n3_bf16_c128(const PrefillArgs& a) {
  return a.out_bf16 ? n3::launch<128, uint16_t>(a) : n3::launch<128, float>(a);
}
#else
hipError_t launch_prefill_n3_bf16_c128(const PrefillArgs& a);

size_t prefill_n3_workspace_floats(int BH, int nseg) {
  if (nseg <= 1) return 0;
  return n3::header_words(BH, nseg) + (size_t)BH * nseg * n3::kImgFloats;
}

hipError_t launch_prefill_n3_bf16(const PrefillArgs& a) {
  switch (a.chunk) {
    case 64: return a.out_bf16 ? n3::launch<64, uint16_t>(a) : n3::launch<64, float>(a);
    case 128: return launch_prefill_n3_bf16_c128(a);
  }
  return hipErrorInvalidValue;
}
#endif

}  // namespace taylor
