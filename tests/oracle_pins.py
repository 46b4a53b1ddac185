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


# Known bf16 bit patterns and the values they encode (bf16 is the top half of
# an IEEE binary32: 1 sign bit, 8 exponent bits with bias 127, 7 fraction
# bits; exponent field 0 = subnormal with scale 2^-126).
BF16_PATTERNS = [
    (0x3F80, 1.0),
    (0xC0A0, -5.0),                       # 1 10000001 0100000: -1.25 * 2^2
    (0x0001, 2.0 ** -133),                # smallest subnormal: 2^-7 * 2^-126
    (0x0080, 2.0 ** -126),                # smallest normal
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),   # largest finite
    (0x3FC0, 1.5),
    (0x4049, 3.140625),                   # 1 + 1/2 + 1/16 + 1/128 = 1.5703125, times 2
    (0xBF80, -1.0),
    (0x0000, 0.0),
]


def bf16_decode_error(decode_fn) -> int:
    """Number of known patterns the decoder gets wrong (sign of zero and the
    infinities included)."""
    bits = np.array([b for b, _ in BF16_PATTERNS] + [0x8000, 0x7F80, 0xFF80], dtype=np.uint16)
    got = np.asarray(decode_fn(bits), dtype=np.float64)
    bad = 0
    for k, (_, want) in enumerate(BF16_PATTERNS):
        bad += int(got[k] != want)
    z, pinf, ninf = got[-3], got[-2], got[-1]
    bad += int(not (z == 0.0 and np.signbit(z)))
    bad += int(not (np.isinf(pinf) and pinf > 0))
    bad += int(not (np.isinf(ninf) and ninf < 0))
    return bad


def nesterov_step_error(step_fn, method: str, shape, beta: float = 0.95) -> float:
    """One step of the whole method from a warm momentum, against the update
    built by hand from the definition:
        m1 = fp32(beta m0 + (1 - beta) g)        (the stored state)
        u  = (1 - beta) g + beta m1              (Nesterov blend)
        X  = u (wide orientation) / (||u||_F + eps)
        update = U f^5(S) V^T * fp32(sqrt(max(1, rows/cols)))
    with U S V^T the SVD of X.  Returns the larger of the update's relative
    error and the momentum's (both should be ~1e-13).  step_fn has the
    oracle's muon_step signature."""
    import math

    import oracle.muon_oracle as O
    rows, cols = shape
    rng = np.random.default_rng(rows * 31 + cols)
    g = rng.standard_normal(shape)
    m0 = (rng.standard_normal(shape) * 3.0).astype(np.float32)   # momentum well away from g's direction
    state = O.MuonState(momenta=[m0.copy()])
    opt = O.MuonOptions(beta=beta, method=method)
    res = step_fn([g], state, [shape], [0], [0], 1, rows * cols, opt)
    m1 = (beta * m0.astype(np.float64) + (1.0 - beta) * g).astype(np.float32)
    u = (1.0 - beta) * g + beta * m1.astype(np.float64)
    x = u.T if rows > cols else u
    x = x / (np.linalg.norm(x) + O.NORM_EPS)
    U, S, Vt = np.linalg.svd(x, full_matrices=False)
    y = (U * quintic(S)) @ Vt
    y = y.T if rows > cols else y
    scale = float(np.float32(math.sqrt(max(1.0, rows / cols))))
    want = y * scale
    got = res.updates[0]
    e_upd = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    e_mom = float(np.max(np.abs(state.momenta[0].astype(np.float64) - m1.astype(np.float64))))
    return max(e_upd, e_mom)
