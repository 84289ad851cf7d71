"""Planted mistakes in the float64 oracle, on the CPU.

Each mutant below is a plausible slip in one of the oracle's C functions: the
direct sum of Eq. (1)-(2) of "A Taylor-Series Route to Linear-Time
Transformers with a Fixed Number of Recurrent States" (section 3.1) with its
dot product and polynomial, exact softmax (Eq. (1)), the |q.k/a| statistics
(section 5.9) and the eviction-fed hybrid of "Tensor Cache:
Eviction-conditioned Associative Memory for Transformers" (sections 3.1-3.2).
The slips: a dropped or mis-weighted term of the polynomial, the temperature
lost or applied twice, a wrong causal bound or window edge, a swapped
operand, a wrong head or token offset, a missing normaliser, a lost absolute
value.  Each is compiled into a library of its own, the oracle is pointed at
it, and at least one of that function's pins (the functions of
test_oracle_pins.py) must fail.  The unchanged source, built the same way,
passes all of them.
"""
import importlib.util
import os
import subprocess
import tempfile

import pytest

import oracle
from oracle import build as obuild

HERE = os.path.dirname(os.path.abspath(__file__))
_spec = importlib.util.spec_from_file_location("oracle_pins", os.path.join(HERE, "test_oracle_pins.py"))
P = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(P)

# (function, description, old text, new text): a mutant applies to one of the
# oracle's C functions (the Taylor direct sum together with the dot product and
# the polynomial it calls) and must match exactly once there
MUTANTS = [
    ("taylor", "drops the highest term of the polynomial", "for (int m = n - 1; m >= 1; --m)",
     "for (int m = n - 2; m >= 1; --m)"),
    ("taylor", "powers without the factorials", "w = 1.0 + w * y / (double)m;", "w = 1.0 + w * y;"),
    ("taylor", "alternating signs", "w = 1.0 + w * y / (double)m;", "w = 1.0 - w * y / (double)m;"),
    ("taylor", "temperature left out", "d) / a, n);", "d), n);"),
    ("taylor", "temperature applied twice", "d) / a, n);", "d) / (a * a), n);"),
    ("taylor", "the query's own key left out", "for (int64_t i = 0; i <= t; ++i) {",
     "for (int64_t i = 0; i < t; ++i) {"),
    ("taylor", "later keys included", "for (int64_t i = 0; i <= t; ++i) {", "for (int64_t i = 0; i < N; ++i) {"),
    ("taylor", "q.q in place of q.k", "dot_f64(qt, kb + (size_t)i * d, d)", "dot_f64(qt, qt, d)"),
    ("taylor", "keys of the first head for every head", "const float* kb = k + (size_t)bh * N * d;",
     "const float* kb = k;"),
    ("taylor", "the query token's value for every key", "const float* vi = vb + (size_t)i * dv;",
     "const float* vi = vb + (size_t)t * dv;"),
    ("taylor", "normaliser left out", "for (int c = 0; c < dv; ++c) out[c] /= z;", "(void)z;"),
    ("taylor", "last dimension of the dot product dropped", "for (int j = 0; j < d; ++j) s +=",
     "for (int j = 0; j < d - 1; ++j) s +="),
    ("softmax", "temperature left out", "exp(dot_f64(qt, kb + (size_t)i * d, d) / a - mx)",
     "exp(dot_f64(qt, kb + (size_t)i * d, d) - mx)"),
    ("softmax", "the query's own key left out", "for (int64_t i = 0; i <= t; ++i) {\n            const double w = exp(",
     "for (int64_t i = 0; i < t; ++i) {\n            const double w = exp("),
    ("softmax", "keys of the first head for every head", "const float* kb = k + (size_t)bh * N * d;",
     "const float* kb = k;"),
    ("softmax", "normaliser left out", "for (int c = 0; c < dv; ++c) out[c] /= z;", "(void)z;"),
    ("arg_stats", "signed instead of absolute arguments", "fabs(dot_f64(qt, kb + (size_t)i * d, d) / a)",
     "(dot_f64(qt, kb + (size_t)i * d, d) / a)"),
    ("arg_stats", "the query's own key left out", "for (int64_t i = 0; i <= t; ++i) {",
     "for (int64_t i = 0; i < t; ++i) {"),
    ("arg_stats", "temperature left out", "d) / a);", "d));"),
    ("hybrid", "window one key too wide", "(i > t - W)", "(i >= t - W)"),
    ("hybrid", "window and memory kernels swapped", "? exp(y) : taylor_weight(y, n)",
     "? taylor_weight(y, n) : exp(y)"),
    ("hybrid", "temperature left out in the window", "? exp(y) :", "? exp(y * a) :"),
    ("hybrid", "normaliser left out", "for (int c = 0; c < dv; ++c) out[c] /= z;", "(void)z;"),
]

# [start, end) of each function's text (the Taylor sum's with its two helpers)
_BOUNDS = {"taylor": ("static double dot_f64(", "void oracle_softmax("),
           "softmax": ("void oracle_softmax(", "void oracle_arg_stats("),
           "arg_stats": ("void oracle_arg_stats(", "void oracle_hybrid_direct("),
           "hybrid": ("void oracle_hybrid_direct(", None)}


def _region(src, fn):
    a, b = _BOUNDS[fn]
    start = src.index(a)
    return start, (src.index(b) if b else len(src))


def _build(tmp, name, src):
    path = os.path.join(tmp, name + ".c")
    with open(path, "w") as f:
        f.write(src)
    lib = os.path.join(tmp, "lib" + name + ".so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", path, "-o", lib, "-lm"], check=True)
    return lib


def _pins(fn):
    return {
        "taylor": [
            P.test_exact_rational_tiny_case,
            lambda: P.test_first_token_returns_its_value(3),
            P.test_one_term_is_running_mean,
            lambda: P.test_direct_equals_recurrence(3, True),
            lambda: P.test_taylor_tends_to_softmax_within_remainder_bound(3, 1.0),
            lambda: P.test_equal_keys_or_large_temperature_give_running_mean(3),
        ],
        "softmax": [
            lambda: P.test_softmax_two_tokens_closed_form(0.7),
            P.test_softmax_equal_keys_and_dominant_key,
            lambda: P.test_taylor_tends_to_softmax_within_remainder_bound(16, 1.0),
        ],
        "arg_stats": [P.test_arg_stats_hand_computed, P.test_arg_stats_matches_brute_force],
        "hybrid": [
            lambda: P.test_hybrid_limits_are_taylor_and_softmax(3),
            lambda: P.test_hybrid_window_partition_closed_form(5),
            P.test_hybrid_error_falls_with_the_window,
        ],
    }[fn]


def _failures(monkeypatch, lib, fn):
    import numpy as np
    monkeypatch.setattr(obuild, "LIB", lib)
    monkeypatch.setattr(oracle, "_LIB", None)
    failed = 0
    old = np.seterr(all="ignore")
    try:
        for pin in _pins(fn):
            try:
                pin()
            except Exception:  # an assertion, or a non-finite value tripping one
                failed += 1
    finally:
        np.seterr(**old)
    return failed


@pytest.fixture(scope="module")
def src():
    with open(obuild.SRC) as f:
        return f.read()


@pytest.mark.parametrize("fn", list(_BOUNDS))
def test_unchanged_source_passes_the_pins(src, monkeypatch, fn):
    with tempfile.TemporaryDirectory() as tmp:
        assert _failures(monkeypatch, _build(tmp, "control", src), fn) == 0


@pytest.mark.parametrize("fn,what,old,new", MUTANTS, ids=[f"{m[0]}: {m[1]}" for m in MUTANTS])
def test_planted_mistake_fails_a_pin(src, monkeypatch, fn, what, old, new):
    s, e = _region(src, fn)
    region = src[s:e]
    assert region.count(old) == 1, f"mutation site of '{what}' not unique in {fn}"
    mutant = src[:s] + region.replace(old, new) + src[e:]
    with tempfile.TemporaryDirectory() as tmp:
        assert _failures(monkeypatch, _build(tmp, "mutant", mutant), fn) >= 1, f"no pin catches ({fn}): {what}"
