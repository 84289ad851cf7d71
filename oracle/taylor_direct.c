/*
 * Float64 CPU oracle for Taylor-state attention -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the bench's CPU-baseline leg may load
 * this file's library.  It shares no code, table or constant with the HIP
 * path and never calls it.
 *
 * Source: "A Taylor-Series Route to Linear-Time Transformers with a Fixed
 * Number of Recurrent States" (arXiv 2610.20637), section 3.1:
 *   Eq. (1)  causal attention o_t = sum_{i<=t} w(q_t,k_i) v_i / sum_{i<=t} w(q_t,k_i)
 *            with w = exp(q.k / a)                          -> oracle_softmax
 *   Eq. (2)  exp(q.k/a) replaced by sum_{m<n} (q.k)^m / (m! a^m)
 *                                                           -> oracle_taylor_direct
 * Everything is the plain O(N^2) definition: no state, no chunking, no
 * reordering.  Inputs are float32 values (exactly representable, e.g. already
 * rounded to bfloat16); all arithmetic is float64; the key loop accumulates
 * sequentially from i = 0 to i = t inclusive; no epsilon or clamp in the
 * division.
 *
 * Layout: q, k [BH, N, d], v [BH, N, dv] contiguous float32.
 * Rows to evaluate: `rows` holds flat indices bh*N + t (nrows of them), or is
 * NULL for all BH*N rows in order.  Output `o` is [nrows, dv] float64; `den`
 * (may be NULL) receives the normaliser of each row.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double dot_f64(const float* x, const float* y, int d) {
    double s = 0.0;
    for (int j = 0; j < d; ++j) s += (double)x[j] * (double)y[j];
    return s;
}

/* Truncated exponential sum_{m=0}^{n-1} y^m / m!, evaluated by Horner's rule
 * in y = x/a:  1 + y(1 + y/2(1 + y/3(...))).  Eq. (2) with alpha_m = 1/(m! a^m). */
static double taylor_weight(double y, int n) {
    double w = 1.0;
    for (int m = n - 1; m >= 1; --m) w = 1.0 + w * y / (double)m;
    return w;
}

/* The kernel values w = p_n(x/a) for an array of scores x (exported so tests
 * can check the polynomial itself: its sign pattern, section 5.10). */
void oracle_taylor_weights(const double* x, int64_t cnt, int n, double a, double* w) {
    for (int64_t i = 0; i < cnt; ++i) w[i] = taylor_weight(x[i] / a, n);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls (timing only; results do not depend on it:
 * every row is summed sequentially by one thread). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

void oracle_taylor_direct(const float* q, const float* k, const float* v,
                          int64_t BH, int64_t N, int d, int dv, int n, double a,
                          const int64_t* rows, int64_t nrows,
                          double* o, double* den) {
    if (rows == NULL) nrows = BH * N;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t flat = rows ? rows[r] : r;
        const int64_t bh = flat / N, t = flat % N;
        const float* qt = q + (size_t)flat * d;
        const float* kb = k + (size_t)bh * N * d;
        const float* vb = v + (size_t)bh * N * dv;
        double* out = o + (size_t)r * dv;
        for (int c = 0; c < dv; ++c) out[c] = 0.0;
        double z = 0.0;
        for (int64_t i = 0; i <= t; ++i) {
            const double w = taylor_weight(dot_f64(qt, kb + (size_t)i * d, d) / a, n);
            const float* vi = vb + (size_t)i * dv;
            for (int c = 0; c < dv; ++c) out[c] += w * (double)vi[c];
            z += w;
        }
        for (int c = 0; c < dv; ++c) out[c] /= z;
        if (den) den[r] = z;
    }
}

/* Exact causal softmax attention, Eq. (1), with the running maximum of the
 * scores subtracted before exponentiation (a rescaling that cancels in the
 * ratio). */
void oracle_softmax(const float* q, const float* k, const float* v,
                    int64_t BH, int64_t N, int d, int dv, double a,
                    const int64_t* rows, int64_t nrows, double* o) {
    if (rows == NULL) nrows = BH * N;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t flat = rows ? rows[r] : r;
        const int64_t bh = flat / N, t = flat % N;
        const float* qt = q + (size_t)flat * d;
        const float* kb = k + (size_t)bh * N * d;
        const float* vb = v + (size_t)bh * N * dv;
        double* out = o + (size_t)r * dv;
        double mx = -INFINITY;
        for (int64_t i = 0; i <= t; ++i) {
            const double s = dot_f64(qt, kb + (size_t)i * d, d) / a;
            if (s > mx) mx = s;
        }
        for (int c = 0; c < dv; ++c) out[c] = 0.0;
        double z = 0.0;
        for (int64_t i = 0; i <= t; ++i) {
            const double w = exp(dot_f64(qt, kb + (size_t)i * d, d) / a - mx);
            const float* vi = vb + (size_t)i * dv;
            for (int c = 0; c < dv; ++c) out[c] += w * (double)vi[c];
            z += w;
        }
        for (int c = 0; c < dv; ++c) out[c] /= z;
    }
}

/* Statistics of the kernel argument x/a = q_t.k_i/a over the causal pairs
 * i <= t of the given rows: max |x/a| and mean |x/a| (section 5.9 reports
 * both to explain non-convergence). */
void oracle_arg_stats(const float* q, const float* k, int64_t BH, int64_t N, int d,
                      double a, const int64_t* rows, int64_t nrows,
                      double* max_abs, double* sum_abs, int64_t* npairs) {
    if (rows == NULL) nrows = BH * N;
    double gmax = 0.0, gsum = 0.0;
    int64_t gcnt = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(max:gmax) reduction(+:gsum,gcnt)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t flat = rows ? rows[r] : r;
        const int64_t bh = flat / N, t = flat % N;
        const float* qt = q + (size_t)flat * d;
        const float* kb = k + (size_t)bh * N * d;
        for (int64_t i = 0; i <= t; ++i) {
            const double y = fabs(dot_f64(qt, kb + (size_t)i * d, d) / a);
            if (y > gmax) gmax = y;
            gsum += y;
            gcnt += 1;
        }
    }
    *max_abs = gmax;
    *sum_abs = gsum;
    *npairs = gcnt;
}

/* Eviction-fed hybrid ("Tensor Cache: Eviction-conditioned Associative
 * Memory for Transformers", sections 3.1-3.2: a FIFO window of the last W
 * key-value pairs read by exact softmax attention, and a memory written only
 * with the pairs the window evicts), with the memory read through the n-term
 * Taylor kernel of the Taylor-state page (Eq. (2) there).  Every earlier token
 * feeds exactly one read path: for row t the keys i > t - W are in the window
 * and weigh exp(q.k/a); the keys i <= t - W have been evicted into the memory
 * and weigh p_n(q.k/a).  Both paths share one normaliser:
 *   o_t = sum_{i<=t} w_i v_i / sum_{i<=t} w_i.
 * W = 0 is the pure Taylor kernel, W >= t + 1 exact softmax.  The plain
 * definition, exp without any shift (the inputs it is used on keep |q.k/a|
 * small). */
void oracle_hybrid_direct(const float* q, const float* k, const float* v,
                          int64_t BH, int64_t N, int d, int dv, int n, double a, int64_t W,
                          const int64_t* rows, int64_t nrows, double* o) {
    if (rows == NULL) nrows = BH * N;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t flat = rows ? rows[r] : r;
        const int64_t bh = flat / N, t = flat % N;
        const float* qt = q + (size_t)flat * d;
        const float* kb = k + (size_t)bh * N * d;
        const float* vb = v + (size_t)bh * N * dv;
        double* out = o + (size_t)r * dv;
        for (int c = 0; c < dv; ++c) out[c] = 0.0;
        double z = 0.0;
        for (int64_t i = 0; i <= t; ++i) {
            const double y = dot_f64(qt, kb + (size_t)i * d, d) / a;
            const double w = (i > t - W) ? exp(y) : taylor_weight(y, n);
            const float* vi = vb + (size_t)i * dv;
            for (int c = 0; c < dv; ++c) out[c] += w * (double)vi[c];
            z += w;
        }
        for (int c = 0; c < dv; ++c) out[c] /= z;
    }
}
