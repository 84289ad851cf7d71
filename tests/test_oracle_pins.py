"""Pins of the float64 oracle against what the paper and the mathematics fix.

Paper: "A Taylor-Series Route to Linear-Time Transformers with a Fixed Number
of Recurrent States" (arXiv 2610.20637).  Printed values come from
tests/golden/pages_figures.json, each with its citation.  Every check here runs
on the CPU; none touches the HIP path.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import taylor_inputs as TI
from oracle import recurrent as R

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _gauss(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# --------------------------------------------------------------------------
# Feature map and state width (sections 3.2 and 3.4, 5.4, 5.7)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("d", [1, 3, 6])
@pytest.mark.parametrize("m", [0, 1, 2, 3, 4])
def test_phi_preserves_inner_product(d, m):
    """<phi_m(q), phi_m(k)> = (q.k)^m = <q^(x)m, k^(x)m> (Eq. (3), section 3.4)."""
    q, k = _gauss(10 + d, d), _gauss(20 + m, d)
    want = float(q @ k) ** m
    full = float(R.tensor_power(q, m) @ R.tensor_power(k, m))
    sym = float(R.phi(q, m) @ R.phi(k, m))
    assert abs(full - want) <= 1e-12 * max(1.0, abs(want))
    assert abs(sym - want) <= 1e-12 * max(1.0, abs(want))


def test_widths_match_printed():
    printed = GOLDEN["symmetric_widths_d16"]["value"]
    assert [len(R.sym_basis(16, m)[0]) for m in range(6)] == printed
    assert [R.width(16, m) for m in range(6)] == printed
    D3 = sum(R.width(16, m) for m in range(3))
    assert D3 * (64 + 1) == GOLDEN["state_elements_per_head_n3"]["value"]


def test_rank_of_tensor_power_span():
    """Rank of span{k^(x)m} over 2,000 Gaussian keys at d = 6 is C(d+m-1, m) (section 5.4)."""
    keys = _gauss(3, 2000, 6)
    for m in range(1, 5):
        M = np.stack([R.tensor_power(k, m) for k in keys])
        s = np.linalg.svd(M, compute_uv=False)
        rank = int(np.sum(s > s[0] * 1e-10))
        assert rank == math.comb(6 + m - 1, m)
        assert rank < 6 ** m or m == 1


def test_svd_truncation_of_order2_state():
    """Order-2 state at d = 6, dv = 24: rank 21 = C(7,2) is lossless, rank 20 is not (Table 4)."""
    assert GOLDEN["svd_order2_lossless_rank"]["value"] == math.comb(7, 2)
    rng = np.random.default_rng(5)
    N, d, dv = 200, 6, 24
    k = _unit(rng.standard_normal((N, d)))
    v = rng.standard_normal((N, dv))
    A2 = sum(np.multiply.outer(R.tensor_power(k[i], 2), np.append(v[i], 1.0)) for i in range(N))
    U, s, Vt = np.linalg.svd(A2, full_matrices=False)
    qs = _unit(rng.standard_normal((16, d)))
    Fq = np.stack([R.tensor_power(x, 2) for x in qs])

    def trunc(r):
        return (U[:, :r] * s[:r]) @ Vt[:r]

    exact = Fq @ A2
    assert np.abs(Fq @ trunc(21) - exact).max() <= 1e-10 * np.abs(exact).max()
    assert np.abs(Fq @ trunc(20) - exact).max() >= 1e-3 * np.abs(exact).max()


# --------------------------------------------------------------------------
# Direct form against the recurrent form (sections 5.1 - 5.3)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("normalise", [False, True])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_direct_equals_recurrence(n, normalise):
    """Recurrent states reproduce the direct truncated kernel at float64 rounding (section 5.1)."""
    printed = GOLDEN["recursion_vs_direct_f64"]["value"]
    rng = np.random.default_rng(100 + n)
    q, k, v = rng.standard_normal((64, 6)), rng.standard_normal((64, 6)), rng.standard_normal((64, 4))
    if normalise:
        q, k = _unit(q), _unit(k)
    q, k, v = (x.astype(np.float32) for x in (q, k, v))
    a = math.sqrt(6)
    direct = oracle.taylor_direct(q, k, v, n, a)
    sym, _ = R.recurrent_attention(q, k, v, n, a, basis="sym")
    assert np.abs(direct - sym).max() <= 100 * printed
    if n <= 4:
        full, _ = R.recurrent_attention(q, k, v, n, a, basis="full")
        assert np.abs(direct - full).max() <= 100 * printed
        # recurrence against rescanning the history (section 5.3): the direct form is the rescan
        assert np.abs(full - sym).max() <= 100 * GOLDEN["recurrence_vs_rescan"]["value"]


def test_additivity_of_states():
    """States on [0,32) + [32,64) equal the state on [0,64); outputs follow (section 5.2)."""
    rng = np.random.default_rng(7)
    q, k, v = (rng.standard_normal(s).astype(np.float32) for s in ((64, 6), (64, 6), (64, 4)))
    a, n = math.sqrt(6), 4
    o_all, s_all = R.recurrent_attention(q, k, v, n, a, basis="full")
    _, s_a = R.recurrent_attention(q[:32], k[:32], v[:32], n, a, basis="full")
    zero = [np.zeros_like(x) for x in s_a]
    _, s_b = R.recurrent_attention(q[32:], k[32:], v[32:], n, a, basis="full", states=zero)
    diff = max(np.abs(x + y - z).max() for x, y, z in zip(s_a, s_b, s_all))
    assert diff <= 100 * GOLDEN["additivity_state"]["value"]
    o_b, _ = R.recurrent_attention(q[32:], k[32:], v[32:], n, a, basis="full", states=s_a)
    assert np.abs(o_b - o_all[32:]).max() <= 100 * GOLDEN["additivity_outputs"]["value"]
    # the direct form continues the same way when the earlier tokens are simply present
    assert np.abs(oracle.taylor_direct(q, k, v, n, a) - o_all).max() <= 1e-13


# --------------------------------------------------------------------------
# Closed forms and special cases of Eq. (1)-(2)
# --------------------------------------------------------------------------
def test_one_term_is_running_mean():
    q, k, v = TI.make_qkv(11, 2, 3, 50, 5, 7)
    o = oracle.taylor_direct(q, k, v, 1, 1.0)
    mean = np.cumsum(v.astype(np.float64), axis=2) / np.arange(1, 51)[:, None]
    assert np.abs(o - mean).max() <= 1e-13


@pytest.mark.parametrize("n", [1, 2, 3, 4, 7])
def test_first_token_returns_its_value(n):
    q, k, v = TI.make_qkv(12, 1, 4, 9, 6, 3, normalize=False)
    o = oracle.taylor_direct(q, k, v, n, 0.7)
    assert np.abs(o[..., 0, :] - v[..., 0, :]).max() <= 1e-15 * 8


@pytest.mark.parametrize("n", [2, 3, 4])
def test_equal_keys_or_large_temperature_give_running_mean(n):
    q, k, v = TI.make_qkv(13, 1, 2, 40, 4, 3)
    mean = np.cumsum(v.astype(np.float64), axis=2) / np.arange(1, 41)[:, None]
    k_eq = np.broadcast_to(k[:, :, :1, :], k.shape).copy()
    assert np.abs(oracle.taylor_direct(q, k_eq, v, n, 1.0) - mean).max() <= 1e-13
    assert np.abs(oracle.taylor_direct(q, k, v, n, 1e12) - mean).max() <= 1e-10


def test_exact_rational_tiny_case():
    """Small-integer inputs: compare against exact rational arithmetic of Eq. (1)-(2)."""
    rng = np.random.default_rng(21)
    N, d, dv, n = 6, 3, 2, 4
    a = Fraction(3, 2)
    q = rng.integers(-2, 3, (N, d)).astype(np.float32)
    k = rng.integers(-2, 3, (N, d)).astype(np.float32)
    v = rng.integers(-3, 4, (N, dv)).astype(np.float32)
    got = oracle.taylor_direct(q, k, v, n, float(a))
    for t in range(N):
        num = [Fraction(0)] * dv
        den = Fraction(0)
        for i in range(t + 1):
            x = sum(Fraction(int(q[t, j])) * Fraction(int(k[i, j])) for j in range(d))
            w = sum((x / a) ** m / math.factorial(m) for m in range(n))
            num = [num[c] + w * int(v[i, c]) for c in range(dv)]
            den += w
        for c in range(dv):
            assert abs(got[t, c] - float(num[c] / den)) <= 1e-14 * max(1.0, abs(float(num[c] / den)))


# --------------------------------------------------------------------------
# The softmax limit (Eq. (1)) and the signs of the truncated kernel
# --------------------------------------------------------------------------
@pytest.mark.parametrize("a", [1.0, 2.5])
@pytest.mark.parametrize("n", [2, 3, 4, 6, 10, 16])
def test_taylor_tends_to_softmax_within_remainder_bound(n, a):
    """|o^(n) - o^soft| <= delta/(1-delta) * max_i |v_i - o^soft| per coordinate, where delta
    bounds |p_n(y) e^-y - 1| over the row's scores; the bound follows from Eq. (1)-(2)."""
    q, k, v = TI.make_qkv(31, 1, 2, 96, 8, 5)
    ref = oracle.softmax(q, k, v, a)
    got = oracle.taylor_direct(q, k, v, n, a)
    for h in range(2):
        x = (q[0, h].astype(np.float64) @ k[0, h].astype(np.float64).T)
        y = x / a
        rel = np.abs(oracle.taylor_weights(x, n, a) * np.exp(-y) - 1.0)
        for t in range(96):
            delta = rel[t, : t + 1].max()
            assert delta < 1
            spread = np.abs(v[0, h, : t + 1].astype(np.float64) - ref[0, h, t]).max(axis=0)
            bound = delta / (1 - delta) * spread
            assert np.all(np.abs(got[0, h, t] - ref[0, h, t]) <= bound * (1 + 1e-9) + 1e-15)
    if n == 16:
        assert np.abs(got - ref).max() <= 1e-12


@pytest.mark.parametrize("a", [0.7, 3.0])
def test_softmax_two_tokens_closed_form(a):
    """Exact softmax (Eq. (1)) with two keys: o_1 = s(d) v_1 + s(-d) v_0 with the logistic
    function s and d = q_1.(k_1 - k_0) / a; o_0 = v_0."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 2, 6)).astype(np.float32)
    k = (2.0 * rng.standard_normal((1, 1, 2, 6))).astype(np.float32)
    v = rng.standard_normal((1, 1, 2, 3)).astype(np.float32)
    got = oracle.softmax(q, k, v, a)[0, 0]
    qq, kk, vv = (x[0, 0].astype(np.float64) for x in (q, k, v))
    d = float(qq[1] @ (kk[1] - kk[0])) / a
    w1 = 1.0 / (1.0 + math.exp(-d))
    assert np.allclose(got[0], vv[0], rtol=0, atol=1e-15)
    assert np.allclose(got[1], w1 * vv[1] + (1.0 - w1) * vv[0], rtol=0, atol=1e-14)


def test_softmax_equal_keys_and_dominant_key():
    """Exact softmax with all keys equal is the running mean of v for any q; a key whose
    score exceeds every other by 60 (e^-60 < 1e-26) takes all the weight."""
    q, k, v = TI.make_qkv(32, 1, 1, 40, 4, 3)
    keq = np.ascontiguousarray(np.broadcast_to(k[:, :, :1], k.shape))
    got = oracle.softmax(q, keq, v, 1.7)[0, 0]
    mean = np.cumsum(v[0, 0].astype(np.float64), axis=0) / np.arange(1, 41)[:, None]
    assert np.abs(got - mean).max() <= 1e-14
    qd = np.zeros((1, 1, 40, 4), np.float32)
    qd[..., 0] = 1.0
    kd = np.zeros((1, 1, 40, 4), np.float32)
    kd[0, 0, 7, 0] = 60.0  # only key 7 scores above 0
    got = oracle.softmax(qd, kd, v, 1.0)[0, 0]
    assert np.abs(got[7:] - v[0, 0, 7].astype(np.float64)).max() <= 1e-20 + 1e-24
    mean7 = np.cumsum(v[0, 0, :7].astype(np.float64), axis=0) / np.arange(1, 8)[:, None]
    assert np.abs(got[:7] - mean7).max() <= 1e-15


def test_negative_kernel_fraction_matches_printed():
    """Fraction of negative kernel values at d = 6, N = 64, a = sqrt(d) (section 5.10)."""
    g = GOLDEN["negative_kernel_fraction"]
    a = math.sqrt(6)
    for n, printed in zip(g["n"], g["value"]):
        fr = []
        for s in range(60):
            rng = np.random.default_rng(s)
            x = rng.standard_normal((64, 6)) @ rng.standard_normal((64, 6)).T
            fr.append(float((oracle.taylor_weights(x, n, a) < 0).mean()))
        if printed == 0.0:
            assert max(fr) == 0.0
        else:
            assert abs(np.mean(fr) - printed) <= 0.1 * printed + 0.003


def test_error_vs_softmax_plausible():
    """n = 3 error against softmax near 6.5e-4 and n = 4 about 18x better (section 5.7)."""
    q, k, v = TI.make_qkv(41, 1, 1, 2048, 16, 64)
    ref = oracle.softmax(q, k, v, 2.0)
    e3 = oracle.rel_err_frobenius(oracle.taylor_direct(q, k, v, 3, 2.0), ref)
    e4 = oracle.rel_err_frobenius(oracle.taylor_direct(q, k, v, 4, 2.0), ref)
    printed = GOLDEN["error_vs_softmax_n3"]["value"]
    assert printed / 3 <= e3 <= printed * 3
    assert 8 <= e3 / e4 <= 40


def test_convergence_report_flags_unnormalised_inputs():
    """Section 5.9: without unit-norm q, k adding terms stops helping; with them it converges."""
    g = GOLDEN["unnormalised_convergence"]
    q, k, v = TI.make_qkv(51, 1, 1, 96, 8, 8, normalize=False)
    rep = oracle.convergence_report(q, k, v, 2.0, 6)
    assert rep["non_converged"]
    assert 0.6 * g["max_arg"] <= rep["max_abs_arg"] <= 1.6 * g["max_arg"]
    assert 0.02 <= rep["err"][5] <= 1.0
    q, k, v = TI.make_qkv(51, 1, 1, 96, 8, 8, normalize=True)
    rep = oracle.convergence_report(q, k, v, 2.0, 6)
    assert not rep["non_converged"]
    assert all(rep["err"][i + 1] < rep["err"][i] for i in range(5))
    q, k, v = TI.make_qkv(51, 1, 1, 96, 8, 8, normalize=False)
    assert oracle.convergence_report(q, k, v, 0.5, 6)["non_converged"]


# --------------------------------------------------------------------------
# Memory closed forms (section 5.8)
# --------------------------------------------------------------------------
def test_memory_closed_forms():
    g = GOLDEN["state_size_bf16_MB"]
    D16 = sum(R.width(16, m) for m in range(6))
    D64 = sum(R.width(64, m) for m in range(6))
    assert round(D16 * 65 * 2 / 2 ** 20, 1) == g["d16_n6"]
    assert round(D64 * 65 * 2 / 2 ** 30, 1) == g["d64_n6_per_head"]
    kv = GOLDEN["kv_cache_bf16_MB"]
    for N, printed in zip(kv["N"], kv["value"]):
        assert round(N * (16 + 64) * 2 / 2 ** 20, 1) == printed


# --------------------------------------------------------------------------
# The input generator (not part of the method, but shared by both sides)
# --------------------------------------------------------------------------
def test_round_bf16_ties_to_even():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -7, -(1 + 2 ** -8) - 2 ** -20, 3.0e38], np.float32)
    want = np.array([1.0, 1.0, 1 + 2 ** -6, 1 + 2 ** -7, -(1 + 2 ** -7), 2.9981e38], np.float32)
    got = TI.round_bf16(x)
    assert np.array_equal(got[:5], want[:5])
    assert np.isfinite(got[5]) and abs(got[5] - 3.0e38) / 3.0e38 < 2 ** -8


def test_inputs_are_seeded_and_per_head():
    q1, k1, v1 = TI.make_qkv(9, 2, 2, 10, 4, 3, dtype="bf16")
    q2, k2, v2 = TI.make_qkv(9, 2, 2, 10, 4, 3, dtype="bf16", heads=[(1, 0)])
    assert np.array_equal(q1[1, 0], q2[1, 0]) and np.array_equal(v1[1, 0], v2[1, 0])
    assert np.array_equal(TI.round_bf16(q1), q1)
    assert np.allclose(np.linalg.norm(q1, axis=-1), 1.0, atol=1e-2)


# --------------------------------------------------------------------------
# The error measures themselves: every GPU parity gate goes through
# rel_err_rowwise, so it is pinned on hand-computed arrays whose value tells
# the row-wise max-norm ratio apart from the plausible slips (a global ratio,
# a mean over rows, the wrong axis, an element-wise ratio, a row 2-norm).
# --------------------------------------------------------------------------
def test_rel_err_rowwise_hand_computed():
    ref = np.array([[1.0, -4.0, 2.0],
                    [0.5, 0.25, -0.5]])
    o = ref + np.array([[0.4, 0.0, 0.0],
                        [0.0, 0.0, -0.1]])
    # row 0: 0.4 / 4 = 0.1; row 1: 0.1 / 0.5 = 0.2 -> max 0.2
    assert oracle.rel_err_rowwise(o, ref) == pytest.approx(0.2, rel=1e-15)
    # the slips give other numbers on the same arrays
    d = np.abs(o - ref)
    assert d.max() / np.abs(ref).max() == pytest.approx(0.1)                           # global ratio
    assert np.mean(d.max(1) / np.abs(ref).max(1)) == pytest.approx(0.15)               # mean over rows
    assert np.max(d.max(0) / np.abs(ref).max(0)) == pytest.approx(0.4)                 # columns as rows
    assert np.max(d / np.abs(ref)) == pytest.approx(0.4)                               # element-wise
    assert np.max(np.linalg.norm(d, axis=1) / np.linalg.norm(ref, axis=1)) != pytest.approx(0.2)
    # symmetric in the sign of the error, scaled by the reference only
    assert oracle.rel_err_rowwise(2 * ref - o, ref) == pytest.approx(0.2, rel=1e-15)
    assert oracle.rel_err_rowwise(o, ref) != pytest.approx(oracle.rel_err_rowwise(ref, o))


def test_rel_err_rowwise_rows_are_last_axis_vectors():
    """[..., d_v] arrays: every leading index is a row; permuting rows does not matter."""
    rng = np.random.default_rng(5)
    ref = rng.standard_normal((2, 3, 4, 5))
    o = ref.copy()
    o[1, 2, 3, 0] += 0.5                      # one element of one row
    want = 0.5 / np.abs(ref[1, 2, 3]).max()
    assert oracle.rel_err_rowwise(o, ref) == pytest.approx(want, rel=1e-15)
    perm = rng.permutation(24)
    assert oracle.rel_err_rowwise(o.reshape(24, 5)[perm], ref.reshape(24, 5)[perm]) == pytest.approx(want, rel=1e-15)
    assert oracle.rel_err_rowwise(ref, ref) == 0.0
    # a non-finite output row is never hidden
    o[0, 0, 0, 1] = np.nan
    assert not oracle.rel_err_rowwise(o, ref) <= 1.0


def test_rel_err_frobenius_hand_computed():
    ref = np.array([[3.0, 0.0], [0.0, 4.0]])            # ||ref||_F = 5
    o = ref + np.array([[0.0, 0.3], [0.4, 0.0]])        # ||o - ref||_F = 0.5
    assert oracle.rel_err_frobenius(o, ref) == pytest.approx(0.1, rel=1e-15)


def test_arg_stats_hand_computed():
    """max and mean of |q_t.k_i / a| over the causal pairs i <= t only (section 5.9)."""
    q = np.array([[[1.0, 0.0], [0.0, -2.0]]], np.float32)
    k = np.array([[[3.0, 0.0], [1.0, 1.0]]], np.float32)
    # pairs (t, i): (0, 0) -> 3/2; (1, 0) -> 0; (1, 1) -> -2/2, |.| = 1
    mx, mean = oracle.arg_stats(q, k, 2.0)
    assert mx == 1.5
    assert mean == pytest.approx((1.5 + 0.0 + 1.0) / 3, rel=1e-15)
    # the non-causal pair (0, 1) = 1/2 and the signed mean would give other values
    assert mean != pytest.approx((1.5 + 0.5 + 0.0 + 1.0) / 4)
    assert mean != pytest.approx((1.5 + 0.0 - 1.0) / 3)
    # a subset of rows: row 1 alone has the pairs (1, 0) and (1, 1)
    mx1, mean1 = oracle.arg_stats(q, k, 2.0, rows=[1])
    assert (mx1, mean1) == (1.0, 0.5)


def test_arg_stats_matches_brute_force():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((3, 7, 4)).astype(np.float32)
    k = rng.standard_normal((3, 7, 4)).astype(np.float32)
    a = 0.7
    vals = [abs(float(np.dot(q[b, t].astype(np.float64), k[b, i].astype(np.float64))) / a)
            for b in range(3) for t in range(7) for i in range(t + 1)]
    mx, mean = oracle.arg_stats(q, k, a)
    assert mx == pytest.approx(max(vals), rel=1e-14)
    assert mean == pytest.approx(sum(vals) / len(vals), rel=1e-13)
    rows = [0, 8, 20]                          # (b, t) = (0, 0), (1, 1), (2, 6)
    sub = [abs(float(np.dot(q[r // 7, r % 7].astype(np.float64), k[r // 7, i].astype(np.float64)))) / a
           for r in rows for i in range(r % 7 + 1)]
    mx2, mean2 = oracle.arg_stats(q, k, a, rows=rows)
    assert mx2 == pytest.approx(max(sub), rel=1e-14)
    assert mean2 == pytest.approx(sum(sub) / len(sub), rel=1e-13)


# --------------------------------------------------------------------------
# The eviction-fed hybrid ("Tensor Cache: Eviction-conditioned Associative
# Memory for Transformers", sections 3.1-3.2, with the Taylor kernel as the
# memory): window keys weigh exp(q.k/a), evicted keys p_n(q.k/a).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("n", [1, 3, 4])
def test_hybrid_limits_are_taylor_and_softmax(n):
    """No window: every key is in the memory (the n-term kernel).  A window as long
    as the sequence: nothing is evicted (exact softmax)."""
    q, k, v = TI.make_qkv(61, 1, 2, 90, 16, 64)
    assert oracle.rel_err_rowwise(oracle.hybrid_direct(q, k, v, n, 1.3, 0), oracle.taylor_direct(q, k, v, n, 1.3)) \
        <= 1e-14
    assert oracle.rel_err_rowwise(oracle.hybrid_direct(q, k, v, n, 1.3, 90), oracle.softmax(q, k, v, 1.3)) <= 1e-13
    assert oracle.rel_err_rowwise(oracle.hybrid_direct(q, k, v, n, 1.3, 500), oracle.softmax(q, k, v, 1.3)) <= 1e-13


@pytest.mark.parametrize("W", [1, 5, 17])
def test_hybrid_window_partition_closed_form(W):
    """All keys equal: row t's score s is the same for every key, so with
    n_w = min(W, t + 1) keys in the window and the other t + 1 - n_w evicted,
    o_t = (e^s * sum_window v + p_n(s) * sum_evicted v) / (n_w e^s + (t + 1 - n_w) p_n(s)).
    An off-by-one in the window boundary changes n_w and fails this."""
    n, a, N = 3, 0.7, 40
    q, k, v = TI.make_qkv(62, 1, 1, N, 8, 5)
    k = np.ascontiguousarray(np.broadcast_to(k[:, :, :1], k.shape))
    got = oracle.hybrid_direct(q, k, v, n, a, W)[0, 0]
    vv = v[0, 0].astype(np.float64)
    for t in range(N):
        s = float(q[0, 0, t].astype(np.float64) @ k[0, 0, 0].astype(np.float64)) / a
        e, p = math.exp(s), 1 + s + s * s / 2
        nw = min(W, t + 1)
        win, ev = vv[t + 1 - nw: t + 1].sum(0), vv[: t + 1 - nw].sum(0)
        want = (e * win + p * ev) / (nw * e + (t + 1 - nw) * p)
        assert np.abs(got[t] - want).max() <= 1e-14 * max(1.0, np.abs(want).max()), t


def test_hybrid_error_falls_with_the_window():
    """With unit-norm q, k the hybrid sits between the n-term kernel and softmax, and
    its error against softmax shrinks as the window grows (plausibility)."""
    q, k, v = TI.make_qkv(63, 1, 1, 600, 16, 64)
    ref = oracle.softmax(q, k, v, 1.0)
    errs = [oracle.rel_err_frobenius(oracle.hybrid_direct(q, k, v, 2, 1.0, W), ref) for W in (0, 64, 256, 599)]
    assert all(errs[i + 1] < errs[i] for i in range(3))
    assert errs[0] == pytest.approx(oracle.rel_err_frobenius(oracle.taylor_direct(q, k, v, 2, 1.0), ref))
