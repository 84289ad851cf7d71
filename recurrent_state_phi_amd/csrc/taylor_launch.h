// Host-side launch interface between the C ABI (taylor_abi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace taylor {

struct DecodeArgs {
  const void* q; const void* k; const void* v; void* o;
  float* state;
  int BH, d, n;
  float a;
  bool in_bf16, out_bf16;
  hipStream_t stream;
};

// How a prefill call is split: every (b, h) sequence is cut into `nseg`
// segments of `chunks_per_seg` chunks of `chunk` tokens.
struct PrefillPlan {
  int nchunks = 0;
  int nseg = 1;
  int chunks_per_seg = 0;
  size_t workspace_floats = 0;  // 0 when nseg == 1
};

PrefillPlan plan_prefill(int BH, int N, int d, int n, int chunk);

struct PrefillArgs {
  const void* q; const void* k; const void* v; void* o;
  float* state;
  float* workspace;
  int BH, N, d, n, chunk;
  float a;
  bool in_bf16, out_bf16;
  PrefillPlan plan;
  hipStream_t stream;
  hipEvent_t* events;  // 4 phase events or nullptr
  int wait_limit;      // polls of a wait between workgroups before it gives up
};

hipError_t launch_decode(const DecodeArgs& a);
// Zero n floats with a kernel (not a memset node, so that a caller may capture
// it in a HIP graph).
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a);

// n = 3, bfloat16 inputs, chunk 64 or 128 (taylor_prefill_n3.hip): one
// launch with a look-back across segments, and the workspace it needs.
hipError_t launch_prefill_n3_bf16(const PrefillArgs& a);
size_t prefill_n3_workspace_floats(int BH, int nseg);
// Header words of that workspace: [1] error code, [2] kN3Magic once the flag-
// clearing kernel has run.
constexpr int kN3Magic = 0x54617933;
constexpr int kN3ErrTimeout = 1;

// n = 1, 2 at d = 16 (taylor_prefill_small.hip): one launch over segments of
// 128 (n = 1) or 256 (n = 2) tokens (16-token chunks inside, whatever the
// requested chunk), with a look-back across segments, and the workspace it
// needs.
hipError_t launch_prefill_small(const PrefillArgs& a);
size_t prefill_small_workspace_floats(int BH, int N, int n);
constexpr int small_segment_tokens(int n) { return n == 1 ? 128 : 256; }

// Test hook (taylor_debug.hip): fills every CU's LDS with `pattern`.
hipError_t launch_fill_lds(uint32_t pattern, hipStream_t stream);

// Feature-blocked prefill, chunk 32 or 64 (taylor_prefill_fb.hip): d = 16
// with n = 3 (one block; bfloat16 inputs with chunk 64 or 128 take the
// single-launch n = 3 kernel instead), 4, 5, 6, and d = 32, 64 with n = 1, 2,
// 3.  The launch, the number of 176-row feature blocks, and the floats of the
// per-block output workspace (none for a single block).
hipError_t launch_prefill_fb(const PrefillArgs& a);
int prefill_fb_blocks(int d, int n);
size_t prefill_fb_output_floats(int BH, int N, int d, int n);

// Exclusive scan of the per-segment state sums in place, seeded with the
// caller's state (taylor_prefill.hip).
hipError_t launch_segment_scan(const float* st_S, const float* st_T, float* W_S, float* W_T, int D, int nseg, int BH,
                               hipStream_t stream);

// Whether a (d, n, chunk, input dtype) combination is compiled.
bool prefill_supported(int d, int n, int chunk, bool in_bf16);

// Exact causal softmax attention (softmax_attn.hip), d = 16, d_v = 64.
struct SoftmaxPrefillArgs {
  const void* q; const void* k; const void* v; void* o;
  int BH, N;
  float a;
  bool in_bf16, out_bf16;
  hipStream_t stream;
};
struct SoftmaxDecodeArgs {
  const void* q; const void* k; const void* v; void* o;
  void* k_cache; void* v_cache;
  float* workspace;
  int BH, pos, cap;
  float a;
  bool in_bf16, out_bf16;
  hipStream_t stream;
};
hipError_t launch_softmax_prefill(const SoftmaxPrefillArgs& a);
hipError_t launch_softmax_decode(const SoftmaxDecodeArgs& a);
// Key ranges of one decode step over `len` keys, and the workspace floats of
// a cache of `cap` positions.
int softmax_decode_splits(int len);
size_t softmax_decode_workspace_floats(int BH, int cap);

// Decode against a bfloat16-stored state with an exact window of recent tokens
// (taylor_decode_bf16.hip), d = 16, d_v = 64, n <= 3.
struct Bf16DecodeArgs {
  const void* q; const void* k; const void* v; void* o;
  void* state;  // bfloat16 S of all heads, then float32 T
  void* win_k; void* win_v;
  int BH, n, step, window;
  float a;
  bool in_bf16, out_bf16;
  hipStream_t stream;
};
hipError_t launch_decode_bf16state(const Bf16DecodeArgs& a);
hipError_t launch_state_to_bf16(const float* state, void* state_bf16, int BH, int D, hipStream_t stream);
int bf16_decode_max_window();

// Eviction-fed hybrid decode (taylor_hybrid.hip), d = 16, d_v = 64, n <= 3.
struct HybridDecodeArgs {
  const void* q; const void* k; const void* v; void* o;
  float* state;
  void* win_k; void* win_v;
  int BH, n, pos, window;
  float a;
  bool in_bf16, out_bf16;
  hipStream_t stream;
};
hipError_t launch_hybrid_decode(const HybridDecodeArgs& a);
hipError_t launch_hybrid_fill_window(const void* k, const void* v, void* wk, void* wv, int BH, int N, int W,
                                     bool in_bf16, hipStream_t stream);
int hybrid_max_window();

}  // namespace taylor
