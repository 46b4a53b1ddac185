"""Checks that pin the oracle to facts other than itself.

Each check takes the function under test as an argument, so that the same
check can be run on the oracle (it must pass) and on copies of the oracle with
a planted mistake (it must fail; see test_oracle_mutations.py).  The facts:

* the scalar picture of the quintic: for X = U S V^T, one Newton-Schulz step
  maps each singular value s to f(s) = a s + b s^3 + c s^5 and keeps U, V, so
  T steps give U f^T(S) V^T (checked against numpy's SVD);
* the Gram form equals the standard form in exact arithmetic;
* closed forms of the momentum recurrence under a constant gradient;
* per-element brute force of the flat-partition index map.
"""

from __future__ import annotations

import numpy as np

COEFFS = (3.4445, -4.7750, 2.0315)


def quintic(s, steps=5, coeffs=COEFFS):
    """f^steps(s) for f(s) = a s + b s^3 + c s^5 (scalar recurrence)."""
    a, b, c = coeffs
    s = np.asarray(s, dtype=np.float64)
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def svd_closed_form_error(ns_fn, x, steps=5, coeffs=COEFFS) -> float:
    """Relative error of ns_fn(x) against U f^T(S) V^T (x already wide and
    normalised)."""
    U, S, Vt = np.linalg.svd(x, full_matrices=False)
    want = (U * quintic(S, steps, coeffs)) @ Vt
    got = ns_fn(x, steps, coeffs)
    return float(np.linalg.norm(got - want) / np.linalg.norm(want))


def gaussian_wide(rng, m, n):
    x = rng.standard_normal((m, n))
    return x / np.linalg.norm(x)


def momentum_closed_form_error(update_fn, beta=0.95, steps=4, nesterov=True) -> float:
    """Constant gradient g from zero momentum: m_t = (1 - beta^t) g, and the
    Nesterov blend u_t = (1 - beta^(t+1)) g (without Nesterov u_t = m_t).
    Returns the largest relative deviation over `steps` steps."""
    g = np.array([[1.0, -2.0, 0.5], [3.0, 0.25, -1.5]])
    m = np.zeros_like(g, dtype=np.float32)
    worst = 0.0
    for t in range(1, steps + 1):
        m, u = update_fn(m, g, beta, nesterov)
        k = t + 1 if nesterov else t
        want_u = (1.0 - beta ** k) * g
        want_m = (1.0 - beta ** t) * g
        worst = max(worst, float(np.max(np.abs(u - want_u) / np.abs(want_u))),
                    float(np.max(np.abs(m - want_m) / np.abs(want_m))))
    return worst


def brute_force_index_map(flat_offset, numel, P):
    """(partition, local offset) of every element, one at a time."""
    out = []
    for j in range(numel):
        f = flat_offset + j
        out.append((f // P, f % P))
    return out


def runs_to_index_map(runs, numel):
    got = [None] * numel
    for r, off, j, n in runs:
        for t in range(n):
            got[j + t] = (r, off + t)
    return got
