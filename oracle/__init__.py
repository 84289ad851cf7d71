"""Float64 CPU oracle for Taylor-state attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path
(``recurrent_state_phi_amd``) and never imports it.

Source of every formula: "A Taylor-Series Route to Linear-Time Transformers
with a Fixed Number of Recurrent States" (arXiv 2610.20637).

* :func:`taylor_direct` -- section 3.1, Eq. (1) with exp replaced by the
  n-term polynomial of Eq. (2); the plain O(N^2) causal sum (C, float64).
* :func:`softmax` -- exact causal softmax, Eq. (1) (C, float64).
* :func:`hybrid_direct` -- the eviction-fed hybrid of "Tensor Cache:
  Eviction-conditioned Associative Memory for Transformers" (sections 3.1-3.2)
  with the Taylor kernel as its memory: exp weights inside the window of the
  last W keys, p_n weights for the evicted keys (C, float64).
* :mod:`oracle.recurrent` -- the recurrent state form of sections 3.2-3.4
  (float64 NumPy), used to pin the direct form and to check exported states.
* :func:`rel_err_rowwise`, :func:`convergence_report` -- the error measures
  and the non-convergence flag used when comparing against softmax.

Pins (tests/test_oracle_pins.py): closed forms (n=1 running mean, t=0, equal
keys, a -> inf), the recurrent form in both the full tensor-power basis and the
symmetric basis, the softmax limit with a pointwise Taylor-remainder bound, the
state widths, rank and SVD bounds of section 5.4, the memory sizes of
section 5.8, the signed-weight fractions of section 5.10, the error measures
and |q.k/a| statistics on hand-computed cases, and the hybrid's two limits and
window partition.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
_i64 = ctypes.c_int64
_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_lp = ctypes.POINTER(ctypes.c_int64)


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.oracle_taylor_direct.argtypes = [_fp, _fp, _fp, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_double, _lp, _i64, _dp, _dp]
        lib.oracle_taylor_direct.restype = None
        lib.oracle_softmax.argtypes = [_fp, _fp, _fp, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_double, _lp, _i64, _dp]
        lib.oracle_softmax.restype = None
        lib.oracle_arg_stats.argtypes = [_fp, _fp, _i64, _i64, ctypes.c_int, ctypes.c_double, _lp,
                                         _i64, _dp, _dp, _lp]
        lib.oracle_arg_stats.restype = None
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        lib.oracle_taylor_weights.argtypes = [_dp, _i64, ctypes.c_int, ctypes.c_double, _dp]
        lib.oracle_taylor_weights.restype = None
        lib.oracle_hybrid_direct.argtypes = [_fp, _fp, _fp, _i64, _i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_double, _i64, _lp, _i64, _dp]
        lib.oracle_hybrid_direct.restype = None
        _LIB = lib
    return _LIB


def num_threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS, else all cores)."""
    return int(_lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the following oracle calls (timing only: each row is summed by one thread)."""
    _lib().oracle_set_num_threads(int(n))


def taylor_weights(x, n: int, a: float):
    """The truncated kernel p_n(x / a) = sum_{m<n} x^m / (m! a^m) for an array of scores x."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    w = np.empty_like(x)
    _lib().oracle_taylor_weights(x.ctypes.data_as(_dp), x.size, int(n), float(a), w.ctypes.data_as(_dp))
    return w


def _prep(q, k, v):
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32) if v is not None else None
    N, d = q.shape[-2], q.shape[-1]
    BH = int(np.prod(q.shape[:-2])) if q.ndim > 2 else 1
    return q, k, v, BH, N, d


def _rows_arg(rows):
    if rows is None:
        return None, None
    r = np.ascontiguousarray(rows, dtype=np.int64).ravel()
    return r, r.ctypes.data_as(_lp)


def taylor_direct(q, k, v, n: int, a: float, rows=None, return_den: bool = False):
    """Causal attention with the n-term Taylor kernel, float64, direct O(N^2) sum.

    q, k: [..., N, d]; v: [..., N, dv] (float32 values, computed in float64).
    rows: optional flat indices ``bh * N + t`` of the query rows to evaluate.
    Returns [..., N, dv] (all rows) or [len(rows), dv] float64.
    """
    q, k, v, BH, N, d = _prep(q, k, v)
    dv = v.shape[-1]
    r, rp = _rows_arg(rows)
    nrows = BH * N if r is None else r.size
    o = np.empty((nrows, dv), np.float64)
    den = np.empty(nrows, np.float64)
    _lib().oracle_taylor_direct(q.ctypes.data_as(_fp), k.ctypes.data_as(_fp), v.ctypes.data_as(_fp),
                                BH, N, d, dv, int(n), float(a), rp, nrows,
                                o.ctypes.data_as(_dp), den.ctypes.data_as(_dp))
    if r is None:
        o = o.reshape(q.shape[:-1] + (dv,))
        den = den.reshape(q.shape[:-1])
    return (o, den) if return_den else o


def softmax(q, k, v, a: float, rows=None):
    """Exact causal softmax attention, float64 (Eq. (1))."""
    q, k, v, BH, N, d = _prep(q, k, v)
    dv = v.shape[-1]
    r, rp = _rows_arg(rows)
    nrows = BH * N if r is None else r.size
    o = np.empty((nrows, dv), np.float64)
    _lib().oracle_softmax(q.ctypes.data_as(_fp), k.ctypes.data_as(_fp), v.ctypes.data_as(_fp),
                          BH, N, d, dv, float(a), rp, nrows, o.ctypes.data_as(_dp))
    if r is None:
        o = o.reshape(q.shape[:-1] + (dv,))
    return o


def hybrid_direct(q, k, v, n: int, a: float, window: int, rows=None):
    """Eviction-fed hybrid, float64, direct O(N^2) sum ("Tensor Cache", sections
    3.1-3.2, with the Taylor-state page's Eq. (2) for the memory): for row t the keys
    i > t - window weigh exp(q.k/a) (the window), the keys i <= t - window weigh
    p_n(q.k/a) (evicted into the memory); one normaliser.  window = 0 is the n-term
    kernel, window >= N exact softmax."""
    q, k, v, BH, N, d = _prep(q, k, v)
    dv = v.shape[-1]
    r, rp = _rows_arg(rows)
    nrows = BH * N if r is None else r.size
    o = np.empty((nrows, dv), np.float64)
    _lib().oracle_hybrid_direct(q.ctypes.data_as(_fp), k.ctypes.data_as(_fp), v.ctypes.data_as(_fp),
                                BH, N, d, dv, int(n), float(a), int(window), rp, nrows, o.ctypes.data_as(_dp))
    if r is None:
        o = o.reshape(q.shape[:-1] + (dv,))
    return o


def arg_stats(q, k, a: float, rows=None):
    """(max |q.k/a|, mean |q.k/a|) over the causal pairs of the given rows."""
    q, k, _, BH, N, d = _prep(q, k, None)
    r, rp = _rows_arg(rows)
    nrows = BH * N if r is None else r.size
    mx, sm, cnt = ctypes.c_double(), ctypes.c_double(), ctypes.c_int64()
    _lib().oracle_arg_stats(q.ctypes.data_as(_fp), k.ctypes.data_as(_fp), BH, N, d, float(a), rp, nrows,
                            ctypes.byref(mx), ctypes.byref(sm), ctypes.byref(cnt))
    return mx.value, sm.value / max(cnt.value, 1)


def rel_err_rowwise(o, ref):
    """max over rows of ||o_t - ref_t||_inf / ||ref_t||_inf (rows = last axis vectors)."""
    o = np.asarray(o, np.float64).reshape(-1, np.shape(o)[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, np.shape(ref)[-1])
    num = np.max(np.abs(o - ref), axis=1)
    den = np.max(np.abs(ref), axis=1)
    return float(np.max(num / den))


def rel_err_frobenius(o, ref):
    """||o - ref||_F / ||ref||_F over the whole array."""
    o = np.asarray(o, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm((o - ref).ravel()) / np.linalg.norm(ref.ravel()))


def convergence_report(q, k, v, a: float, n_max: int = 6, rows=None):
    """Error of the n-term kernel against exact softmax for n = 1..n_max.

    Section 5.9 of the paper: without unit-norm q, k the argument q.k/a leaves
    the range where the truncated series helps, and adding terms stops reducing
    the error.  ``non_converged`` is set when err(n+1) >= err(n) for some n, or
    when err(n_max) > 1e-2.
    """
    ref = softmax(q, k, v, a, rows=rows)
    errs = [rel_err_frobenius(taylor_direct(q, k, v, n, a, rows=rows), ref) for n in range(1, n_max + 1)]
    mx, mean = arg_stats(q, k, a, rows=rows)
    stalls = any(errs[i + 1] >= errs[i] for i in range(len(errs) - 1))
    return {
        "err": errs,
        "max_abs_arg": mx,
        "mean_abs_arg": mean,
        "non_converged": bool(stalls or errs[-1] > 1e-2),
    }
