"""Float64 recurrent-state form of Taylor-state attention -- TEST INFRASTRUCTURE ONLY.

Written from "A Taylor-Series Route to Linear-Time Transformers with a Fixed
Number of Recurrent States" (arXiv 2610.20637):

* section 3.2, Eq. (3): (q.k)^m = <q^{(x)m}, k^{(x)m}>  -> :func:`tensor_power`
* section 3.3, Eq. (6)-(7): one state per order, A_m(t) = A_m(t-1) + k_t^{(x)m} (x) [v_t; 1],
  read out as Eq. (5)                                     -> :func:`recurrent_attention`
* section 3.4: the symmetric basis of nondecreasing multi-indices with weight
  sqrt(m! / prod_i c_i!), c_i the multiplicity of coordinate i -> :func:`sym_basis`, :func:`phi`

Slow and plain: one Python-level loop over tokens, NumPy for the per-token
outer products.  Used to pin :func:`oracle.taylor_direct` (the two must agree to
rounding) and to check the states the GPU path exports.  The state of order m
is returned as a (D_m, d_v + 1) array: rows are the basis features, the last
column is the ones-column (the normaliser T_m of Eq. (4)).
"""
from __future__ import annotations

import itertools
import math

import numpy as np

__all__ = ["sym_basis", "phi", "tensor_power", "width", "recurrent_attention", "state_rows"]


def width(d: int, m: int) -> int:
    """Number of distinct monomials of degree m in d variables, C(d+m-1, m)."""
    return math.comb(d + m - 1, m)


def sym_basis(d: int, m: int):
    """Nondecreasing multi-indices of length m over range(d), lexicographic, and their weights.

    The weight of a multi-index with coordinate multiplicities c_0..c_{d-1} is
    sqrt(m! / prod c_i!), so that <phi_m(q), phi_m(k)> = (q.k)^m (section 3.4).
    """
    idx = list(itertools.combinations_with_replacement(range(d), m))
    w = []
    for t in idx:
        counts = [t.count(i) for i in set(t)]
        w.append(math.sqrt(math.factorial(m) / math.prod(math.factorial(c) for c in counts)))
    return idx, np.asarray(w, np.float64)


def phi(x: np.ndarray, m: int) -> np.ndarray:
    """Symmetric-basis features phi_m(x) of shape [..., C(d+m-1, m)] in float64."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    idx, w = sym_basis(d, m)
    out = np.empty(x.shape[:-1] + (len(idx),), np.float64)
    for j, t in enumerate(idx):
        val = np.ones(x.shape[:-1], np.float64)
        for i in t:
            val = val * x[..., i]
        out[..., j] = w[j] * val
    return out


def tensor_power(x: np.ndarray, m: int) -> np.ndarray:
    """The full tensor power x^{(x)m} of one vector, flattened to length d^m (Eq. (3))."""
    x = np.asarray(x, np.float64)
    out = np.ones(1, np.float64)
    for _ in range(m):
        out = np.multiply.outer(out, x).ravel()
    return out


def recurrent_attention(q, k, v, n: int, a: float, basis: str = "sym", states=None):
    """Outputs of one head by the per-token recurrence of Eq. (7) and readout of Eq. (5).

    q, k: [N, d]; v: [N, dv].  ``basis`` is "sym" (section 3.4) or "full"
    (uncompressed tensor powers, Eq. (3)).  ``states`` is an optional list of
    initial states A_m (one per m < n); they are added to, as in Eq. (7).
    Returns (o [N, dv], states).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N, d = q.shape
    dv = v.shape[1]
    feat = (lambda x, m: phi(x, m)) if basis == "sym" else (lambda x, m: tensor_power(x, m))
    if states is None:
        states = [np.zeros((width(d, m) if basis == "sym" else d ** m, dv + 1)) for m in range(n)]
    else:
        states = [np.array(s, np.float64, copy=True) for s in states]
    alpha = [1.0 / (math.factorial(m) * a ** m) for m in range(n)]
    o = np.empty((N, dv))
    for t in range(N):
        vt = np.append(v[t], 1.0)                                   # [v; 1], Eq. (6)
        for m in range(n):
            states[m] += np.multiply.outer(feat(k[t], m), vt)       # Eq. (7), update first (i <= t)
        y = sum(alpha[m] * (feat(q[t], m) @ states[m]) for m in range(n))   # Eq. (5)
        o[t] = y[:dv] / y[dv]
    return o, states


def state_rows(states):
    """Concatenate the per-order states (m ascending) into one (D, dv+1) array."""
    return np.concatenate(states, axis=0)
