/*
 * taylor_attn.h -- C ABI of the MI355X (gfx950) Taylor-state attention library.
 *
 * Method: "A Taylor-Series Route to Linear-Time Transformers with a Fixed Number
 * of Recurrent States" (arXiv 2610.20637).
 *   section 3.1, Eq. (1)-(2): causal attention with exp(q.k/a) replaced by the
 *       n-term polynomial sum_{m<n} (q.k)^m / (m! a^m);
 *   section 3.2-3.3, Eq. (3)-(7): the history collapses into n states
 *       A_m = sum_i k_i^{(x)m} (x) [v_i; 1], one rank-one update per token;
 *   section 3.4: each state stored in the symmetric basis of C(d+m-1, m)
 *       monomials with weights sqrt(m! / prod_i c_i!);
 *   section 3.5: prefill in chunks -- a causally masked c x c block on the
 *       diagonal plus the states for everything earlier; states are additive.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Supported shapes: d_v = 64 with d = 16 and n in {1, ..., 6} (state widths
 *   D = 1, 17, 153, 969, 4845, 20349), or d = 32, 64 and n in {1, 2, 3}
 *   (D = 1, 33, 561 and 1, 65, 2145); section 5.8 discusses both directions.
 *   Anything else returns TAYLOR_EUNSUPPORTED without launching.
 * - Tensors are dense, row-major, on the current HIP device:
 *     q, k : [B, H, N, d]       v, o : [B, H, N, d_v]      (decode: N = 1)
 *   element type given by `in_dtype` (q, k, v) and `out_dtype` (o).
 * - State (float32, B*H*taylor_state_numel(d, d_v, n) floats, one buffer):
 *     first  B*H*D*d_v floats: S[b][h][D][d_v]   (value index fastest)
 *     then   B*H*D     floats: T[b][h][D]        (the ones-column, Eq. (6))
 *   with D = taylor_state_width(d, n).  Row r enumerates the features of all
 *   orders m = 0..n-1 in ascending m; inside one order the multi-indices
 *   i_1 <= ... <= i_m appear in lexicographic order; every row carries the
 *   sqrt-multinomial weight of section 3.4.  The temperature a and the factors
 *   1/(m! a^m) are applied when the state is read, so the state does not
 *   depend on a.
 * - Prefill and decode ADD to the state they are given (Eq. (7)): output o_t
 *   sees the tokens already folded into `state` plus this call's tokens i <= t.
 *   Prefill of [0, N) equals prefill of [0, t1) followed by prefill of [t1, N),
 *   and equals N single-token decode calls (up to rounding).
 * - No normalisation of q or k happens inside; the division by the normaliser
 *   has no epsilon and no clamp.
 * - Ownership: the caller owns every buffer.  The library never allocates
 *   device memory and never synchronises (taylor_prefill_check aside, which
 *   exists to wait for a result); all work is enqueued on `stream`
 *   (0 = the null stream).  Calls are thread-safe; the error string is
 *   thread-local.
 * - Errors: TAYLOR_EINVAL (bad pointer or size, nothing launched),
 *   TAYLOR_EUNSUPPORTED (shape or option not built, nothing launched),
 *   TAYLOR_EHIP (a HIP call failed; the message names it),
 *   TAYLOR_ETIMEOUT (from taylor_prefill_check only: a bounded wait between
 *   workgroups ran out).
 *   taylor_last_error() describes the last failure on the calling thread.
 */
#ifndef TAYLOR_ATTN_H
#define TAYLOR_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;

typedef enum { TAYLOR_F32 = 0, TAYLOR_BF16 = 1 } taylor_dtype;

enum {
    TAYLOR_OK = 0,
    TAYLOR_EINVAL = -1,
    TAYLOR_EUNSUPPORTED = -2,
    TAYLOR_EHIP = -3,
    TAYLOR_ETIMEOUT = -4
};

/* D = sum_{m<n} C(d+m-1, m): rows of the stacked state (section 3.4; Eq. (6)
 * stacked over m).  Host only.  Returns -1 for d < 1 or n < 1. */
int64_t taylor_state_width(int d, int n);

/* Floats per (b, h) head: D * (d_v + 1) (section 4, "Memory").  Host only.
 * Returns -1 for invalid arguments. */
int64_t taylor_state_numel(int d, int d_v, int n);

/* Zero B*H heads of state (the empty history, Eq. (4) at t < 0), with a
 * kernel (no memset node, so the call may be captured in a HIP graph).
 * state: device, B*H*taylor_state_numel(d, d_v, n) floats. */
int taylor_state_init(float* state, int B, int H, int d, int d_v, int n, hipStream_t stream);

/* Bytes of device workspace taylor_attn_prefill needs for these sizes (0 when
 * the sequence fits one segment and the state one 176-row block, i.e. D <= 176).
 * Host only; -1 cast to size_t on
 * error.  For states of several 176-row feature blocks (d = 16 with n >= 4,
 * and n = 3 at d = 32, 64) it includes a row of d_v + 4 floats per
 * head-token per feature block.  For n = 1, 2 at d = 16 (segments of 128
 * tokens for n = 1 and 256 for n = 2, so 0 for N up to one segment) it is a
 * 64-word header, one flag word per
 * segment rounded up to 64 words, and two state images per segment of 1,108
 * (n = 2) or 68 (n = 1) floats; `chunk` does not change it. */
size_t taylor_prefill_workspace_bytes(int B, int H, int N, int d, int d_v, int n, int chunk);

/* Chunked prefill (section 3.5): for every head and every t in [0, N)
 *   o_t = sum_m alpha_m <phi_m(q_t), A_m(t)>[:d_v] / (same)[d_v],
 *   A_m(t) = state_m + sum_{i<=t} phi_m(k_i) [v_i; 1]^T          (Eq. (5)-(7))
 * evaluated in chunks of `chunk` tokens: the masked chunk x chunk polynomial
 * block on the diagonal, the states for all earlier tokens.  On return (in
 * stream order) `state` holds A_m(N-1).
 *   q, k, v : device, in_dtype (TAYLOR_F32 or TAYLOR_BF16); o : device, out_dtype.
 *   N >= 0 (N = 0 is a no-op), any N (the last chunk may be partial).
 *   a > 0 : temperature.
 *   chunk : d = 16, n = 1..3: 32 or 64 for TAYLOR_F32 inputs; 32, 64 or 128
 *           for TAYLOR_BF16.  d = 16 with n = 4..6, and d = 32, 64: 32 or 64
 *           for either input type.  At d = 16 with n = 1, 2 the value is
 *           checked but the kernel always evaluates chunks of 16 tokens inside
 *           segments of 128 (n = 1) or 256 (n = 2) tokens (the outputs agree
 *           to float32 rounding).
 *   Arithmetic: float32 inputs use float32 MFMA throughout.  bfloat16 inputs
 *   use bfloat16 MFMA with float32 accumulation and a float32 state at d = 16
 *   for n = 3 with chunk 64 or 128; everywhere else (d = 16 with n = 1, 2, n =
 *   3 with chunk 32, d = 16 with n = 4..6, d = 32 and 64) they are widened
 *   and computed in float32.  Those float32 paths split the state into
 *   blocks of 176 rows handled by separate workgroups (1 block for n = 3 at
 *   d = 16; 6, 28, 116 blocks for n = 4, 5, 6; 4 and 13 for n = 3 at d = 32,
 *   64); with more than one block the workspace also holds each block's share
 *   of the outputs.
 *   workspace : device, at least taylor_prefill_workspace_bytes(...) bytes
 *   (may be NULL when that is 0); it is scratch, its contents are undefined
 *   afterwards (any contents are fine on entry).  o must not alias q, k, v or
 *   state.
 *   n = 1, 2 at d = 16 and n = 3 with bfloat16 inputs (chunk 64 or 128) run
 *   as one kernel in which the workgroups of a sequence's segments pass their
 *   state sums to each other through the workspace; every such wait is
 *   bounded, and taylor_prefill_check reports whether one ran out.  Which
 *   sums each segment adds, and in which order, depends only on the sizes, so
 *   repeated calls give the same bits. */
int taylor_attn_prefill(const void* q, const void* k, const void* v, void* o, float* state,
                        int B, int H, int N, int d, int d_v, int n, float a, int chunk,
                        taylor_dtype in_dtype, taylor_dtype out_dtype,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* taylor_attn_prefill for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and results without the workspace.  Its
 * scratch is a fixed 32 MiB device array, one per GPU the library runs on,
 * held until the process ends; this call allocates nothing and calls no
 * allocating routine.  A plan that needs more (taylor_prefill_workspace_bytes
 * > 32 MiB: d = 16 with n >= 4, whose per-block partial outputs are large,
 * the wide heads, and n = 1, 2 at d = 16 beyond about 3,780 segments of 256
 * tokens (n = 2) or 61,000 segments of 128 tokens (n = 1) over all heads) returns
 * TAYLOR_EINVAL with the size in the message and launches nothing; every
 * plan with n = 3 at d = 16 fits.  All calls on one
 * GPU share its array: calls that overlap in time on one GPU (other streams,
 * other threads) race and must be serialised by the caller.  Whatever a call
 * leaves in the array is cleared or overwritten by the next before it is
 * read.  A time-out of a wait between workgroups cannot be queried for this
 * variant (taylor_prefill_check needs the workspace pointer). */
int taylor_attn_prefill_noalloc(const void* q, const void* k, const void* v, void* o, float* state,
                                int B, int H, int N, int d, int d_v, int n, float a, int chunk,
                                taylor_dtype in_dtype, taylor_dtype out_dtype, hipStream_t stream);

/* One decode step per head (section 3.3, Eq. (7), then Eq. (5)): update the
 * state with the new token first, then read it (the token attends to itself).
 *   q, k : device [B, H, d]; v, o : device [B, H, d_v]; dtypes as above.
 *   state: device, read and written in place. */
int taylor_attn_decode(const void* q, const void* k, const void* v, void* o, float* state,
                       int B, int H, int d, int d_v, int n, float a,
                       taylor_dtype in_dtype, taylor_dtype out_dtype, hipStream_t stream);

/* ---- bfloat16 state storage (section 5.8 sizes the states in bfloat16) -----
 * A state whose S part (the D x d_v block) is kept in bfloat16, with T (the
 * ones-column, D floats) in float32, and decode steps against it.  Rounding the
 * state after every token would lose most tokens' increments (a row of S sums
 * the whole context, one token's term is below half a bfloat16 unit of it), so
 * the last tokens are kept exactly in a window of K (k, v) pairs, read with the
 * same weights p_n(q.k / a) as the state, and folded into the bfloat16 S once
 * every K tokens (one rounding per K tokens).  Outputs are the n-term Taylor
 * attention of Eq. (5) over all keys; the bfloat16 base is the only lossy part.
 * Built for d = 16, d_v = 64, n <= 3, 1 <= K <= 128.
 * Layout of a bfloat16 state (16-byte aligned, device): S[B][H][D][d_v] as
 * bfloat16 (value index fastest, rows and weights as in the float32 state),
 * then T[B][H][D] as float32.  Window: win_k [B, H, K, d], win_v [B, H, K, d_v]
 * in in_dtype, caller-owned; its contents between folds belong to the state. */

/* Bytes per head of a bfloat16 state: D * d_v * 2 + D * 4.  Host only; -1 on
 * invalid arguments. */
int64_t taylor_state_bf16_bytes(int d, int d_v, int n);

/* Round a float32 state (e.g. after a prefill) to the bfloat16 layout above
 * (round to nearest even; T copied).  The window starts empty (step 0). */
int taylor_state_to_bf16(const float* state, void* state_bf16, int B, int H, int d, int d_v, int n,
                         hipStream_t stream);

/* One decode step against a bfloat16 state.  `step` (0 <= step < window) is
 * the number of tokens in the window since the last fold; the call writes the
 * token (k, v) into window slot `step`, computes
 *   o = (phi_hat(q) [S | T] + sum_{j <= step} p_n(q.k_j / a) [v_j; 1])[:d_v] / (same)[d_v],
 * and when step == window - 1 folds the window into the state (the next call
 * then passes step 0).  Every stream of the batch is at the same step.  No
 * workspace; allocates nothing. */
int taylor_attn_decode_bf16state(const void* q, const void* k, const void* v, void* o, void* state_bf16,
                                 void* win_k, void* win_v, int step, int window, int B, int H, int d, int d_v,
                                 int n, float a, taylor_dtype in_dtype, taylor_dtype out_dtype,
                                 hipStream_t stream);

/* ---- Eviction-fed hybrid ------------------------------------------------------
 * "Tensor Cache: Eviction-conditioned Associative Memory for Transformers"
 * (sections 3.1-3.2): a FIFO window of the last W key-value pairs read by
 * exact softmax, and a memory written only with the pairs the window evicts;
 * here the memory is the n-term Taylor state above (that page fuses its two
 * paths with a learned gate; without training, both paths share one
 * normaliser).  For the token at position t:
 *   o_t = (sum_{t-W < i <= t} e^{q.k_i/a} [v_i; 1] + phi_hat(q_t) A)[:d_v] / (same)[d_v],
 * A = the float32 state of the tokens i <= t - W (layout as above).  W = 1 ..
 * 1024, d = 16, d_v = 64, n <= 3.  Window ring: win_k [B, H, W, d], win_v
 * [B, H, W, d_v] in in_dtype; position i lives in slot i % W. */

/* Fill the ring from a context of N tokens (k, v [B, H, N, d / d_v]): its last
 * min(N, W) tokens go to their slots.  Together with a prefill of the first
 * max(0, N - W) tokens into the state, this is the hybrid's state after N
 * tokens. */
int taylor_hybrid_fill_window(const void* k, const void* v, void* win_k, void* win_v, int B, int H, int N,
                              int window, int d, int d_v, taylor_dtype in_dtype, hipStream_t stream);

/* One decode step at position pos (the number of earlier tokens; all streams
 * alike): the token at pos - W (if pos >= W) leaves the window and is added to
 * the state (write-on-evict, Eq. (7) of the Taylor-state page); the new token
 * takes its slot; o is computed as above.  No workspace. */
int taylor_hybrid_decode(const void* q, const void* k, const void* v, void* o, float* state, void* win_k,
                         void* win_v, int pos, int window, int B, int H, int d, int d_v, int n, float a,
                         taylor_dtype in_dtype, taylor_dtype out_dtype, hipStream_t stream);

/* ---- Exact causal softmax attention: the comparison method ---------------
 * Eq. (1) with the exponential kernel itself, o_t = sum_{i<=t} e^{q_t.k_i/a} v_i /
 * sum_{i<=t} e^{q_t.k_i/a}: what the paper measures the Taylor states against
 * (prefill, section 5.5; decode against a growing key-value cache, section
 * 5.6; accuracy of the n-term kernel, sections 5.7 and 5.9).  Computed with
 * the running maximum subtracted inside the exponential (a factor that
 * cancels in the ratio).  Only d = 16, d_v = 64 are built (else
 * TAYLOR_EUNSUPPORTED, nothing launched).
 *   bfloat16 inputs: bfloat16 matrix-core operands, the weights rounded to
 *   bfloat16 for the weighted sum of v and the normaliser summed from the same
 *   rounded weights, float32 accumulation.  float32 inputs: float32
 *   throughout. */

/* Causal softmax attention over q, k, v [B, H, N, d / d_v] (no earlier
 * context); o [B, H, N, d_v] in out_dtype.  Allocates nothing, needs no
 * workspace.  N = 0 or B*H = 0 is a no-op. */
int taylor_softmax_prefill(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d, int d_v,
                           float a, taylor_dtype in_dtype, taylor_dtype out_dtype, hipStream_t stream);

/* Bytes of workspace taylor_softmax_decode needs for a cache of `cap`
 * positions (one partial result of 68 floats per head per range of 2048
 * keys).  Host only; -1 cast to size_t on invalid arguments. */
size_t taylor_softmax_decode_workspace_bytes(int B, int H, int cap, int d, int d_v);

/* One decode step of every head against its key-value cache (section 5.6).
 *   k_cache [B, H, cap, d], v_cache [B, H, cap, d_v], in_dtype, device: positions
 *   0 .. pos-1 hold the earlier tokens; the call writes k, v ([B, H, d],
 *   [B, H, d_v]) at position pos and then computes o [B, H, d_v] for q
 *   [B, H, d] over positions 0 .. pos (the token attends to itself).
 *   Every stream of the batch is at the same position.  0 <= pos < cap.
 *   workspace: device, at least taylor_softmax_decode_workspace_bytes(B, H,
 *   pos + 1, ...) bytes, 16-byte aligned, scratch. */
int taylor_softmax_decode(const void* q, const void* k, const void* v, void* o, void* k_cache, void* v_cache, int B,
                          int H, int pos, int cap, int d, int d_v, float a, taylor_dtype in_dtype,
                          taylor_dtype out_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Description of the last failure on the calling thread ("" if none). */
const char* taylor_last_error(void);

/* Profiling hook.  With count == 4 and non-NULL events, every following
 * taylor_attn_prefill on this thread records events[0] before its first
 * launch, events[1] after the segment-sum kernel, events[2] after the scan
 * kernel and events[3] after the chunk kernel, all on its stream (events of
 * phases that do not run are recorded back to back).  For the single-kernel
 * paths (n = 1, 2 at d = 16; n = 3 with bfloat16 inputs) events[1] follows
 * the small kernel that clears the workspace flags and events[2], events[3]
 * are recorded by the prefill kernel's dispatch itself, at its start and its
 * end.
 * count == 0 turns it off.  The events stay owned by the caller. */
int taylor_set_phase_events(hipEvent_t* events, int count);

/* Outcome of the waits between workgroups in the last taylor_attn_prefill that
 * used `workspace` (n = 1, 2 at d = 16, or n = 3 with bfloat16 inputs, with
 * more than one segment per sequence).  Waits for the work queued on `stream` (the one call here that
 * synchronises), then returns TAYLOR_OK, or TAYLOR_ETIMEOUT if a wait ran
 * out, in which case that call's outputs and state are wrong.  A workspace
 * that such a call did not use (NULL, too small, or last used by another
 * path) gives TAYLOR_OK.  A wait can only run out if the device stalls a
 * running workgroup for longer than the limit (a workgroup only waits for
 * workgroups that started before it). */
int taylor_prefill_check(const void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Test hook for the time-out path: the number of polls (each followed by a
 * short sleep) after which a wait between workgroups gives up; default
 * 1 << 20 (at least 0.4 s).  Process-wide; returns the previous value, or -1
 * for a negative argument (nothing changed). */
int taylor_set_wait_limit(int polls);

/* Test hook for reads of LDS before it is written (races between the waves of
 * a workgroup, a missing initialisation): fills the LDS of every CU with the
 * 32-bit `pattern` (0xFFFFFFFF reads as a float NaN, 0 re-zeros it) by a
 * kernel on `stream`, so that the next kernel on that stream starts from LDS
 * holding it.  Results of every entry point must not depend on it.  Returns
 * TAYLOR_EHIP if the launch fails. */
int taylor_debug_fill_lds(unsigned int pattern, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TAYLOR_ATTN_H */
