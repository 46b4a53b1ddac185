"""Plant plausible mistakes in copies of the oracle's functions (on the CPU)
and check that the pins catch each of them."""

from __future__ import annotations

import numpy as np
import pytest

import oracle.muon_oracle as O
from oracle_pins import (brute_force_index_map, gaussian_wide, momentum_closed_form_error,
                         runs_to_index_map, svd_closed_form_error)


def _std_drop_square(x, steps=5, coeffs=O.NS_COEFFS):
    a, b, c = coeffs
    for _ in range(steps):
        A = x @ x.T
        x = a * x + (b * A + c * A) @ x
    return x


def _std_wrong_sign(x, steps=5, coeffs=O.NS_COEFFS):
    a, b, c = coeffs
    for _ in range(steps):
        A = x @ x.T
        x = a * x - (b * A + c * (A @ A)) @ x
    return x


def _std_transposed_operand(x, steps=5, coeffs=O.NS_COEFFS):
    a, b, c = coeffs
    for _ in range(steps):
        A = x @ x  # should be x @ x.T
        x = a * x + (b * A + c * (A @ A)) @ x
    return x


def _std_coeff_order(x, steps=5, coeffs=O.NS_COEFFS):
    a, b, c = coeffs
    return O.ns_standard(x, steps, (a, c, b))


def _gram_one_sided(x0, steps=5, coeffs=O.NS_COEFFS):
    a, b, c = coeffs
    eye = np.eye(x0.shape[0])
    R, Q = x0 @ x0.T, eye.copy()
    for k in range(1, steps + 1):
        P = a * eye + b * R + c * (R @ R)
        Q = P @ Q
        if k < steps:
            R = P @ R  # should be P R P
    return Q @ x0


def _gram_stale_r(x0, steps=5, coeffs=O.NS_COEFFS):
    a, b, c = coeffs
    eye = np.eye(x0.shape[0])
    R, Q = x0 @ x0.T, eye.copy()
    for _ in range(steps):
        P = a * eye + b * R + c * (R @ R)
        Q = P @ Q
    return Q @ x0


@pytest.mark.parametrize("bad", [_std_drop_square, _std_wrong_sign, _std_coeff_order,
                                 _gram_one_sided, _gram_stale_r])
def test_svd_pin_catches_ns_mistakes(bad):
    rng = np.random.default_rng(3)
    x = gaussian_wide(rng, 9, 17)
    assert svd_closed_form_error(bad, x) > 1e-3


def test_svd_pin_catches_transposed_operand():
    rng = np.random.default_rng(4)
    x = gaussian_wide(rng, 8, 8)
    assert svd_closed_form_error(_std_transposed_operand, x) > 1e-3


def _mom_swapped_beta(m, g, beta, nesterov):
    return O.momentum_update(m, g, 1.0 - beta, nesterov)


def _mom_nesterov_old_state(m, g, beta, nesterov):
    m_new, _ = O.momentum_update(m, g, beta, False)
    u = (1.0 - beta) * g + beta * np.asarray(m, dtype=np.float64)
    return m_new, (u if nesterov else m_new.astype(np.float64))


def _mom_no_decay(m, g, beta, nesterov):
    m_new = (np.asarray(m, np.float64) + (1.0 - beta) * g).astype(np.float32)
    u = (1.0 - beta) * g + beta * m_new if nesterov else m_new.astype(np.float64)
    return m_new, u


@pytest.mark.parametrize("bad", [_mom_swapped_beta, _mom_nesterov_old_state, _mom_no_decay])
def test_momentum_pin_catches_mistakes(bad):
    assert momentum_closed_form_error(bad, 0.95, 4, True) > 1e-3


def _runs_off_by_one(flat_offset, numel, P):
    runs, j = [], 0
    while j < numel:
        r, off = divmod(flat_offset + j + 1, P)
        n = min(numel - j, P - off)
        if n <= 0:
            n = 1
        runs.append((r, off, j, n))
        j += n
    return runs


def test_layout_pin_catches_index_mistake():
    assert runs_to_index_map(_runs_off_by_one(5, 40, 16), 40) != brute_force_index_map(5, 40, 16)
    assert runs_to_index_map(O.partition_runs(5, 40, 16), 40) == brute_force_index_map(5, 40, 16)


# ------------------------------------------- clipping and the param update


def _clip_no_clamp(norm, max_norm):
    return 1.0 if max_norm <= 0 else max_norm / (norm + O.CLIP_EPS)


def _clip_inverted(norm, max_norm):
    return 1.0 if max_norm <= 0 else min(1.0, (norm + O.CLIP_EPS) / max_norm)


@pytest.mark.parametrize("bad", [_clip_no_clamp, _clip_inverted])
def test_clip_pins_catch_mistakes(bad, monkeypatch):
    monkeypatch.setattr(O, "clip_coefficient", bad)
    import test_oracle_pins as T
    with pytest.raises(AssertionError):
        T.test_clip_coefficient_cases()
        T.test_apply_update_clipped_step_has_max_norm()


_APPLY = O.apply_update


def _apply_wrong_sign(params, partitions, shapes, offsets, lr, weight_decay, max_norm, skip=False):
    return _APPLY(params, partitions, shapes, offsets, -lr, -weight_decay, max_norm, skip)


def _apply_coupled_decay(params, partitions, shapes, offsets, lr, weight_decay, max_norm, skip=False):
    # decay applied to the update instead of the parameter
    out, norm, clip = _APPLY(params, partitions, shapes, offsets, lr, 0.0, max_norm, skip)
    return [o * np.float32(1.0 - lr * weight_decay) for o in out], norm, clip


@pytest.mark.parametrize("bad", [_apply_wrong_sign, _apply_coupled_decay])
def test_apply_pins_catch_mistakes(bad, monkeypatch):
    monkeypatch.setattr(O, "apply_update", bad)
    import test_oracle_pins as T
    with pytest.raises(AssertionError):
        T.test_apply_update_closed_forms()
