// C ABI of the Taylor-state attention library: argument checks, workspace
// sizing and dispatch to the gfx950 kernels.  Declarations and the contract
// of every entry point are in include/taylor_attn.h.
#include "../../include/taylor_attn.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <mutex>
#include <string>

#include "taylor_device.h"
#include "taylor_launch.h"

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_phase_events[4] = {nullptr, nullptr, nullptr, nullptr};
thread_local bool g_phase_events_on = false;
std::atomic<int> g_wait_limit{1 << 20};

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int64_t binom(int64_t n, int64_t k) {
  int64_t r = 1;
  for (int64_t i = 1; i <= k; ++i) r = r * (n - k + i) / i;
  return r;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shapes compiled into this build: d_v = 64 with d = 16 and n = 1..6, or
// d = 32, 64 and n = 1..3.
bool shape_supported(int d, int d_v, int n) {
  if (d_v != taylor::kDV || n < 1) return false;
  return (d == taylor::kD && n <= 6) || ((d == 32 || d == 64) && n <= 3);
}

int check_dtypes(taylor_dtype in, taylor_dtype out) {
  if ((in != TAYLOR_F32 && in != TAYLOR_BF16) || (out != TAYLOR_F32 && out != TAYLOR_BF16))
    return fail(TAYLOR_EINVAL, "dtype must be TAYLOR_F32 or TAYLOR_BF16");
  return TAYLOR_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(TAYLOR_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

// ---- the prefill's scratch for callers that cannot allocate ------------------
// One fixed array per device, held until the process ends.  In host code the
// name `scratch` is only a stand-in for the symbol: its device address comes
// from hipGetSymbolAddress, once per device (with that device current), and
// only that address is ever handed to kernels.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array, or nullptr (message set).
void* device_scratch(int* code) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *code = hip_fail(e, "taylor_attn_prefill_noalloc: hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *code = fail(TAYLOR_EUNSUPPORTED, "taylor_attn_prefill_noalloc: device index beyond 63");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      *code = hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                       "taylor_attn_prefill_noalloc: hipGetSymbolAddress(scratch)");
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int64_t taylor_state_width(int d, int n) {
  if (d < 1 || n < 1) return -1;
  int64_t s = 0;
  for (int m = 0; m < n; ++m) s += binom(d + m - 1, m);
  return s;
}

int64_t taylor_state_numel(int d, int d_v, int n) {
  if (d_v < 1) return -1;
  const int64_t D = taylor_state_width(d, n);
  return D < 0 ? -1 : D * (int64_t)(d_v + 1);
}

const char* taylor_last_error(void) { return g_last_error.c_str(); }

int taylor_set_phase_events(hipEvent_t* events, int count) {
  if (count == 0) {
    g_phase_events_on = false;
    return TAYLOR_OK;
  }
  if (count != 4 || events == nullptr) return fail(TAYLOR_EINVAL, "taylor_set_phase_events: need 4 events or count 0");
  for (int i = 0; i < 4; ++i) {
    if (events[i] == nullptr) return fail(TAYLOR_EINVAL, "taylor_set_phase_events: null event");
    g_phase_events[i] = events[i];
  }
  g_phase_events_on = true;
  return TAYLOR_OK;
}

int taylor_state_init(float* state, int B, int H, int d, int d_v, int n, hipStream_t stream) {
  if (B < 0 || H < 0) return fail(TAYLOR_EINVAL, "taylor_state_init: B and H must be >= 0");
  if (!shape_supported(d, d_v, n)) return fail(TAYLOR_EUNSUPPORTED, "taylor_state_init: only d_v=64 with d=16, n in 1..6 or d=32/64, n in 1..3");
  const size_t floats = (size_t)B * H * taylor_state_numel(d, d_v, n);
  if (floats == 0) return TAYLOR_OK;
  if (state == nullptr) return fail(TAYLOR_EINVAL, "taylor_state_init: state is NULL");
  const hipError_t e = taylor::launch_fill_zero(state, floats, stream);
  if (e != hipSuccess) return hip_fail(e, "taylor_state_init: kernel launch");
  return TAYLOR_OK;
}

size_t taylor_prefill_workspace_bytes(int B, int H, int N, int d, int d_v, int n, int chunk) {
  if (B < 0 || H < 0 || N < 0 || !shape_supported(d, d_v, n) || chunk <= 0) return (size_t)-1;
  const taylor::PrefillPlan p = taylor::plan_prefill(B * H, N, d, n, chunk);
  return p.workspace_floats * sizeof(float);
}

int taylor_attn_prefill(const void* q, const void* k, const void* v, void* o, float* state, int B, int H, int N,
                        int d, int d_v, int n, float a, int chunk, taylor_dtype in_dtype, taylor_dtype out_dtype,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (int e = check_dtypes(in_dtype, out_dtype)) return e;
  if (B < 0 || H < 0 || N < 0) return fail(TAYLOR_EINVAL, "taylor_attn_prefill: B, H, N must be >= 0");
  if (!(a > 0.0f) || a == __builtin_inff()) return fail(TAYLOR_EINVAL, "taylor_attn_prefill: a must be finite and > 0");
  if (!shape_supported(d, d_v, n))
    return fail(TAYLOR_EUNSUPPORTED, "taylor_attn_prefill: only d_v=64 with d=16, n in 1..6 or d=32/64, n in 1..3 are built");
  const bool in_bf16 = in_dtype == TAYLOR_BF16, out_bf16 = out_dtype == TAYLOR_BF16;
  if (!taylor::prefill_supported(d, n, chunk, in_bf16))
    return fail(TAYLOR_EUNSUPPORTED, "taylor_attn_prefill: unsupported (d, n, chunk, in_dtype): at d = 16, n in 1..3, "
                                     "chunk must be 32/64 (float32) or 32/64/128 (bfloat16); otherwise 32/64");
  if ((int64_t)B * H == 0 || N == 0) return TAYLOR_OK;
  if (!q || !k || !v || !o || !state) return fail(TAYLOR_EINVAL, "taylor_attn_prefill: NULL tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(state))
    return fail(TAYLOR_EINVAL, "taylor_attn_prefill: q, k, v, o and state must be 16-byte aligned");
  if ((int64_t)B * H > (1 << 24) || (int64_t)N * chunk > ((int64_t)1 << 40))
    return fail(TAYLOR_EINVAL, "taylor_attn_prefill: sizes out of range");
  // n <= 2 at d = 16: one workgroup per segment (256 threads per 128 tokens at
  // n = 1, 512 per 256 at n = 2)
  if (d == 16 && n <= 2 &&
      (int64_t)B * H * ((N + taylor::small_segment_tokens(n) - 1) / taylor::small_segment_tokens(n)) >= (1 << 23))
    return fail(TAYLOR_EINVAL, "taylor_attn_prefill: sizes out of range (B*H*ceil(N/" +
                                   std::to_string(taylor::small_segment_tokens(n)) + ") must be < 2^23 for n = " +
                                   std::to_string(n) + ")");
  const taylor::PrefillPlan plan = taylor::plan_prefill(B * H, N, d, n, chunk);
  const size_t need = plan.workspace_floats * sizeof(float);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need)
      return fail(TAYLOR_EINVAL, "taylor_attn_prefill: workspace too small (need " + std::to_string(need) +
                                     " bytes, see taylor_prefill_workspace_bytes)");
    if (!aligned16(workspace)) return fail(TAYLOR_EINVAL, "taylor_attn_prefill: workspace must be 16-byte aligned");
  }
  taylor::PrefillArgs args{q, k, v, o, state, static_cast<float*>(workspace), B * H, N, d, n, chunk, a,
                           in_bf16, out_bf16, plan, stream, g_phase_events_on ? g_phase_events : nullptr,
                           g_wait_limit.load(std::memory_order_relaxed)};
  const hipError_t e = taylor::launch_prefill(args);
  if (e != hipSuccess) return hip_fail(e, "taylor_attn_prefill: kernel launch");
  return TAYLOR_OK;
}

int taylor_attn_prefill_noalloc(const void* q, const void* k, const void* v, void* o, float* state, int B, int H,
                                int N, int d, int d_v, int n, float a, int chunk, taylor_dtype in_dtype,
                                taylor_dtype out_dtype, hipStream_t stream) {
  // Anything taylor_attn_prefill rejects, or does without a workspace, goes
  // there unchanged (same checks, same messages, nothing launched on error);
  // then the plan's workspace size is checked against the fixed scratch.
  const bool bad = check_dtypes(in_dtype, out_dtype) != TAYLOR_OK || B < 0 || H < 0 || N < 0 || !(a > 0.0f) ||
                   a == __builtin_inff() || !shape_supported(d, d_v, n) ||
                   !taylor::prefill_supported(d, n, chunk, in_dtype == TAYLOR_BF16) || (int64_t)B * H == 0 ||
                   N == 0 || !q || !k || !v || !o || !state || !aligned16(q) || !aligned16(k) || !aligned16(v) ||
                   !aligned16(o) || !aligned16(state) || (int64_t)B * H > (1 << 24);
  if (bad)
    return taylor_attn_prefill(q, k, v, o, state, B, H, N, d, d_v, n, a, chunk, in_dtype, out_dtype, nullptr, 0,
                               stream);
  const size_t need = taylor::plan_prefill(B * H, N, d, n, chunk).workspace_floats * sizeof(float);
  if (need > kScratchBytes)
    return fail(TAYLOR_EINVAL, "taylor_attn_prefill_noalloc: this call needs " + std::to_string(need) +
                                   " bytes of workspace; the fixed scratch holds " + std::to_string(kScratchBytes) +
                                   " (use taylor_attn_prefill with a workspace)");
  if (need == 0)
    return taylor_attn_prefill(q, k, v, o, state, B, H, N, d, d_v, n, a, chunk, in_dtype, out_dtype, nullptr, 0,
                               stream);
  int code = TAYLOR_OK;
  void* ws = device_scratch(&code);
  if (ws == nullptr) return code;
  return taylor_attn_prefill(q, k, v, o, state, B, H, N, d, d_v, n, a, chunk, in_dtype, out_dtype, ws,
                             kScratchBytes, stream);
}

int taylor_attn_decode(const void* q, const void* k, const void* v, void* o, float* state, int B, int H, int d,
                       int d_v, int n, float a, taylor_dtype in_dtype, taylor_dtype out_dtype, hipStream_t stream) {
  if (int e = check_dtypes(in_dtype, out_dtype)) return e;
  if (B < 0 || H < 0) return fail(TAYLOR_EINVAL, "taylor_attn_decode: B and H must be >= 0");
  if (!(a > 0.0f) || a == __builtin_inff()) return fail(TAYLOR_EINVAL, "taylor_attn_decode: a must be finite and > 0");
  if (!shape_supported(d, d_v, n))
    return fail(TAYLOR_EUNSUPPORTED, "taylor_attn_decode: only d_v=64 with d=16, n in 1..6 or d=32/64, n in 1..3 are built");
  if ((int64_t)B * H == 0) return TAYLOR_OK;
  if ((int64_t)B * H > (1 << 30)) return fail(TAYLOR_EINVAL, "taylor_attn_decode: B*H out of range");
  if (!q || !k || !v || !o || !state) return fail(TAYLOR_EINVAL, "taylor_attn_decode: NULL tensor pointer");
  if (!aligned16(state) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(TAYLOR_EINVAL, "taylor_attn_decode: q, k, v, o and state must be 16-byte aligned");
  taylor::DecodeArgs args{q, k, v, o, state, B * H, d, n, a, in_dtype == TAYLOR_BF16, out_dtype == TAYLOR_BF16,
                          stream};
  const hipError_t e = taylor::launch_decode(args);
  if (e != hipSuccess) return hip_fail(e, "taylor_attn_decode: kernel launch");
  return TAYLOR_OK;
}

int taylor_prefill_check(const void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (workspace == nullptr || workspace_bytes < 3 * sizeof(int)) return TAYLOR_OK;
  int hdr[3] = {0, 0, 0};
  hipError_t e = hipMemcpyAsync(hdr, workspace, sizeof(hdr), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "taylor_prefill_check");
  if (hdr[2] != taylor::kN3Magic || hdr[1] == 0) return TAYLOR_OK;
  return fail(TAYLOR_ETIMEOUT, "taylor_prefill_check: a wait between workgroups ran out; that call's outputs and "
                               "state are wrong");
}

int taylor_set_wait_limit(int polls) {
  if (polls < 0) return fail(TAYLOR_EINVAL, "taylor_set_wait_limit: polls must be >= 0"), -1;
  return g_wait_limit.exchange(polls);
}

int taylor_debug_fill_lds(unsigned int pattern, hipStream_t stream) {
  if (hipError_t e = taylor::launch_fill_lds(pattern, stream))
    return fail(TAYLOR_EHIP, std::string("taylor_debug_fill_lds: ") + hipGetErrorString(e));
  return TAYLOR_OK;
}

int taylor_softmax_prefill(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d, int d_v,
                           float a, taylor_dtype in_dtype, taylor_dtype out_dtype, hipStream_t stream) {
  if (int e = check_dtypes(in_dtype, out_dtype)) return e;
  if (B < 0 || H < 0 || N < 0) return fail(TAYLOR_EINVAL, "taylor_softmax_prefill: B, H, N must be >= 0");
  if (!(a > 0.0f) || a == __builtin_inff()) return fail(TAYLOR_EINVAL, "taylor_softmax_prefill: a must be finite and > 0");
  if (d != taylor::kD || d_v != taylor::kDV)
    return fail(TAYLOR_EUNSUPPORTED, "taylor_softmax_prefill: only d = 16, d_v = 64 are built");
  if ((int64_t)B * H == 0 || N == 0) return TAYLOR_OK;
  if (!q || !k || !v || !o) return fail(TAYLOR_EINVAL, "taylor_softmax_prefill: NULL tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(TAYLOR_EINVAL, "taylor_softmax_prefill: q, k, v and o must be 16-byte aligned");
  if ((int64_t)B * H * ((N + 63) / 64) > ((int64_t)1 << 31) - 1 || (int64_t)N * d_v * 4 > ((int64_t)1 << 31) - 1)
    return fail(TAYLOR_EINVAL, "taylor_softmax_prefill: sizes out of range");
  taylor::SoftmaxPrefillArgs args{q, k, v, o, B * H, N, a, in_dtype == TAYLOR_BF16, out_dtype == TAYLOR_BF16, stream};
  const hipError_t e = taylor::launch_softmax_prefill(args);
  if (e != hipSuccess) return hip_fail(e, "taylor_softmax_prefill: kernel launch");
  return TAYLOR_OK;
}

size_t taylor_softmax_decode_workspace_bytes(int B, int H, int cap, int d, int d_v) {
  if (B < 0 || H < 0 || cap < 1 || d != taylor::kD || d_v != taylor::kDV) return (size_t)-1;
  return taylor::softmax_decode_workspace_floats(B * H, cap) * sizeof(float);
}

int taylor_softmax_decode(const void* q, const void* k, const void* v, void* o, void* k_cache, void* v_cache, int B,
                          int H, int pos, int cap, int d, int d_v, float a, taylor_dtype in_dtype,
                          taylor_dtype out_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (int e = check_dtypes(in_dtype, out_dtype)) return e;
  if (B < 0 || H < 0) return fail(TAYLOR_EINVAL, "taylor_softmax_decode: B and H must be >= 0");
  if (cap < 1 || pos < 0 || pos >= cap) return fail(TAYLOR_EINVAL, "taylor_softmax_decode: need 0 <= pos < cap");
  if (!(a > 0.0f) || a == __builtin_inff()) return fail(TAYLOR_EINVAL, "taylor_softmax_decode: a must be finite and > 0");
  if (d != taylor::kD || d_v != taylor::kDV)
    return fail(TAYLOR_EUNSUPPORTED, "taylor_softmax_decode: only d = 16, d_v = 64 are built");
  if ((int64_t)B * H == 0) return TAYLOR_OK;
  if (!q || !k || !v || !o || !k_cache || !v_cache) return fail(TAYLOR_EINVAL, "taylor_softmax_decode: NULL pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return fail(TAYLOR_EINVAL, "taylor_softmax_decode: tensors must be 16-byte aligned");
  const size_t need = taylor::softmax_decode_workspace_floats(B * H, pos + 1) * sizeof(float);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
    return fail(TAYLOR_EINVAL, "taylor_softmax_decode: workspace too small or unaligned (need " +
                                   std::to_string(need) + " bytes, see taylor_softmax_decode_workspace_bytes)");
  if ((int64_t)B * H * taylor::softmax_decode_splits(pos + 1) > ((int64_t)1 << 31) - 1)
    return fail(TAYLOR_EINVAL, "taylor_softmax_decode: sizes out of range");
  taylor::SoftmaxDecodeArgs args{q, k, v, o, k_cache, v_cache, static_cast<float*>(workspace), B * H, pos, cap, a,
                                 in_dtype == TAYLOR_BF16, out_dtype == TAYLOR_BF16, stream};
  const hipError_t e = taylor::launch_softmax_decode(args);
  if (e != hipSuccess) return hip_fail(e, "taylor_softmax_decode: kernel launch");
  return TAYLOR_OK;
}

int64_t taylor_state_bf16_bytes(int d, int d_v, int n) {
  if (d_v < 1) return -1;
  const int64_t D = taylor_state_width(d, n);
  return D < 0 ? -1 : D * (int64_t)d_v * 2 + D * 4;
}

int taylor_state_to_bf16(const float* state, void* state_bf16, int B, int H, int d, int d_v, int n,
                         hipStream_t stream) {
  if (B < 0 || H < 0) return fail(TAYLOR_EINVAL, "taylor_state_to_bf16: B and H must be >= 0");
  if (d != taylor::kD || d_v != taylor::kDV || n < 1 || n > 3)
    return fail(TAYLOR_EUNSUPPORTED, "taylor_state_to_bf16: only d = 16, d_v = 64, n <= 3 are built");
  if ((int64_t)B * H == 0) return TAYLOR_OK;
  if (!state || !state_bf16) return fail(TAYLOR_EINVAL, "taylor_state_to_bf16: NULL pointer");
  if (!aligned16(state) || !aligned16(state_bf16))
    return fail(TAYLOR_EINVAL, "taylor_state_to_bf16: buffers must be 16-byte aligned");
  const hipError_t e = taylor::launch_state_to_bf16(state, state_bf16, B * H, (int)taylor_state_width(d, n), stream);
  if (e != hipSuccess) return hip_fail(e, "taylor_state_to_bf16: kernel launch");
  return TAYLOR_OK;
}

int taylor_attn_decode_bf16state(const void* q, const void* k, const void* v, void* o, void* state_bf16,
                                 void* win_k, void* win_v, int step, int window, int B, int H, int d, int d_v,
                                 int n, float a, taylor_dtype in_dtype, taylor_dtype out_dtype, hipStream_t stream) {
  if (int e = check_dtypes(in_dtype, out_dtype)) return e;
  if (B < 0 || H < 0) return fail(TAYLOR_EINVAL, "taylor_attn_decode_bf16state: B and H must be >= 0");
  if (!(a > 0.0f) || a == __builtin_inff())
    return fail(TAYLOR_EINVAL, "taylor_attn_decode_bf16state: a must be finite and > 0");
  if (d != taylor::kD || d_v != taylor::kDV || n < 1 || n > 3)
    return fail(TAYLOR_EUNSUPPORTED, "taylor_attn_decode_bf16state: only d = 16, d_v = 64, n <= 3 are built");
  if (window < 1 || window > taylor::bf16_decode_max_window() || step < 0 || step >= window)
    return fail(TAYLOR_EINVAL, "taylor_attn_decode_bf16state: need 1 <= window <= " +
                                   std::to_string(taylor::bf16_decode_max_window()) + " and 0 <= step < window");
  if ((int64_t)B * H == 0) return TAYLOR_OK;
  if ((int64_t)B * H > (1 << 30)) return fail(TAYLOR_EINVAL, "taylor_attn_decode_bf16state: B*H out of range");
  if (!q || !k || !v || !o || !state_bf16 || !win_k || !win_v)
    return fail(TAYLOR_EINVAL, "taylor_attn_decode_bf16state: NULL pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(state_bf16) ||
      !aligned16(win_k) || !aligned16(win_v))
    return fail(TAYLOR_EINVAL, "taylor_attn_decode_bf16state: buffers must be 16-byte aligned");
  taylor::Bf16DecodeArgs args{q, k, v, o, state_bf16, win_k, win_v, B * H, n, step, window, a,
                              in_dtype == TAYLOR_BF16, out_dtype == TAYLOR_BF16, stream};
  const hipError_t e = taylor::launch_decode_bf16state(args);
  if (e != hipSuccess) return hip_fail(e, "taylor_attn_decode_bf16state: kernel launch");
  return TAYLOR_OK;
}

int taylor_hybrid_fill_window(const void* k, const void* v, void* win_k, void* win_v, int B, int H, int N, int window,
                              int d, int d_v, taylor_dtype in_dtype, hipStream_t stream) {
  if (in_dtype != TAYLOR_F32 && in_dtype != TAYLOR_BF16)
    return fail(TAYLOR_EINVAL, "taylor_hybrid_fill_window: dtype must be TAYLOR_F32 or TAYLOR_BF16");
  if (B < 0 || H < 0 || N < 0) return fail(TAYLOR_EINVAL, "taylor_hybrid_fill_window: B, H, N must be >= 0");
  if (d != taylor::kD || d_v != taylor::kDV)
    return fail(TAYLOR_EUNSUPPORTED, "taylor_hybrid_fill_window: only d = 16, d_v = 64 are built");
  if (window < 1 || window > taylor::hybrid_max_window())
    return fail(TAYLOR_EINVAL, "taylor_hybrid_fill_window: need 1 <= window <= " +
                                   std::to_string(taylor::hybrid_max_window()));
  if ((int64_t)B * H == 0 || N == 0) return TAYLOR_OK;
  if ((int64_t)B * H > 65535) return fail(TAYLOR_EINVAL, "taylor_hybrid_fill_window: B*H out of range (<= 65535)");
  if (!k || !v || !win_k || !win_v) return fail(TAYLOR_EINVAL, "taylor_hybrid_fill_window: NULL pointer");
  const hipError_t e = taylor::launch_hybrid_fill_window(k, v, win_k, win_v, B * H, N, window, in_dtype == TAYLOR_BF16,
                                                         stream);
  if (e != hipSuccess) return hip_fail(e, "taylor_hybrid_fill_window: kernel launch");
  return TAYLOR_OK;
}

int taylor_hybrid_decode(const void* q, const void* k, const void* v, void* o, float* state, void* win_k, void* win_v,
                         int pos, int window, int B, int H, int d, int d_v, int n, float a, taylor_dtype in_dtype,
                         taylor_dtype out_dtype, hipStream_t stream) {
  if (int e = check_dtypes(in_dtype, out_dtype)) return e;
  if (B < 0 || H < 0) return fail(TAYLOR_EINVAL, "taylor_hybrid_decode: B and H must be >= 0");
  if (!(a > 0.0f) || a == __builtin_inff()) return fail(TAYLOR_EINVAL, "taylor_hybrid_decode: a must be finite and > 0");
  if (d != taylor::kD || d_v != taylor::kDV || n < 1 || n > 3)
    return fail(TAYLOR_EUNSUPPORTED, "taylor_hybrid_decode: only d = 16, d_v = 64, n <= 3 are built");
  if (window < 1 || window > taylor::hybrid_max_window() || pos < 0)
    return fail(TAYLOR_EINVAL, "taylor_hybrid_decode: need 1 <= window <= " +
                                   std::to_string(taylor::hybrid_max_window()) + " and pos >= 0");
  if ((int64_t)B * H == 0) return TAYLOR_OK;
  if ((int64_t)B * H > (1 << 30)) return fail(TAYLOR_EINVAL, "taylor_hybrid_decode: B*H out of range");
  if (!q || !k || !v || !o || !state || !win_k || !win_v) return fail(TAYLOR_EINVAL, "taylor_hybrid_decode: NULL pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(state) || !aligned16(win_k) ||
      !aligned16(win_v))
    return fail(TAYLOR_EINVAL, "taylor_hybrid_decode: buffers must be 16-byte aligned");
  taylor::HybridDecodeArgs args{q, k, v, o, state, win_k, win_v, B * H, n, pos, window, a,
                                in_dtype == TAYLOR_BF16, out_dtype == TAYLOR_BF16, stream};
  const hipError_t e = taylor::launch_hybrid_decode(args);
  if (e != hipSuccess) return hip_fail(e, "taylor_hybrid_decode: kernel launch");
  return TAYLOR_OK;
}

}  // extern "C"
