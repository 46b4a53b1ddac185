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


# --------------------------------------------- bf16 decoding, parity metric


def _bf16_shift15(bits):
    u32 = bits.astype(np.uint32) << np.uint32(15)
    return u32.view(np.float32).astype(np.float64)


def _bf16_as_fp16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _bf16_low_half(bits):
    # value placed in the low half of the fp32 word instead of the high half
    return np.asarray(bits, dtype=np.uint16).astype(np.uint32).view(np.float32).astype(np.float64)


def _bf16_unsigned(bits):
    return np.abs(O.bf16_bits_to_f64(bits))


@pytest.mark.parametrize("bad", [_bf16_shift15, _bf16_as_fp16, _bf16_low_half, _bf16_unsigned])
def test_bf16_pin_catches_decode_mistakes(bad):
    from oracle_pins import bf16_decode_error
    assert bf16_decode_error(bad) > 0


def _rel_by_got(got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    den = np.linalg.norm(got)
    num = np.linalg.norm(got - want)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def _rel_max_abs(got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    den = np.max(np.abs(want)) if want.size else 0.0
    num = np.max(np.abs(got - want)) if want.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def _rel_zero_want_is_zero(got, want):
    want = np.asarray(want, np.float64)
    if np.linalg.norm(want) == 0.0:
        return 0.0
    return _REL(got, want)


_REL = O.rel_frobenius


def _rel_nan_on_zero(got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        return float(np.linalg.norm(got - want) / np.linalg.norm(want))


@pytest.mark.parametrize("bad", [_rel_by_got, _rel_max_abs, _rel_zero_want_is_zero, _rel_nan_on_zero])
def test_metric_pin_catches_mistakes(bad, monkeypatch):
    monkeypatch.setattr(O, "rel_frobenius", bad)
    import test_oracle_pins as T
    with pytest.raises(AssertionError):
        T.test_rel_frobenius_hand_values()


# ------------------------------------------- the step's Nesterov wiring


def _step_feeds_momentum(grads, state, shapes, heads, offsets, num_partitions, partition_numel, opt,
                         partitions=None, grad_scale=1.0, skip=False):
    """muon_step with the stored momentum, not the Nesterov blend, handed to
    Newton-Schulz."""
    res = O.StepResult()
    res.partitions = partitions or [np.zeros(partition_numel, dtype=np.float32) for _ in range(num_partitions)]
    for i, (rows, cols) in enumerate(shapes):
        g = np.asarray(grads[i], dtype=np.float64).reshape(rows, cols) * float(grad_scale)
        m_new, _u = O.momentum_update(state.momenta[i], g, opt.beta, opt.nesterov)
        state.momenta[i] = m_new
        y = O.muon_matrix_update(m_new.astype(np.float64), opt.method, heads[i], opt.steps, opt.coeffs, opt.eps)
        res.updates.append(y * O.shape_scale(rows, cols))
    return res


def _step_blends_old_momentum(grads, state, shapes, heads, offsets, num_partitions, partition_numel, opt,
                              partitions=None, grad_scale=1.0, skip=False):
    """Nesterov blend formed with the momentum before this step's update."""
    res = O.StepResult()
    for i, (rows, cols) in enumerate(shapes):
        g = np.asarray(grads[i], dtype=np.float64).reshape(rows, cols)
        m_old = state.momenta[i].astype(np.float64)
        m_new, _ = O.momentum_update(state.momenta[i], g, opt.beta, opt.nesterov)
        state.momenta[i] = m_new
        u = (1.0 - opt.beta) * g + opt.beta * m_old
        y = O.muon_matrix_update(u, opt.method, heads[i], opt.steps, opt.coeffs, opt.eps)
        res.updates.append(y * O.shape_scale(rows, cols))
    return res


def _step_no_shape_scale(grads, state, shapes, heads, offsets, num_partitions, partition_numel, opt,
                         partitions=None, grad_scale=1.0, skip=False):
    res = O.muon_step(grads, state, shapes, heads, offsets, num_partitions, partition_numel, opt)
    rows, cols = shapes[0]
    res.updates = [u / O.shape_scale(rows, cols) for u in res.updates]
    return res


@pytest.mark.parametrize("bad", [_step_feeds_momentum, _step_blends_old_momentum])
@pytest.mark.parametrize("method", ["standard", "gram"])
def test_step_pin_catches_wiring_mistakes(bad, method):
    from oracle_pins import nesterov_step_error
    assert nesterov_step_error(bad, method, (9, 17)) > 1e-4


def test_step_pin_catches_missing_shape_scale():
    from oracle_pins import nesterov_step_error
    assert nesterov_step_error(_step_no_shape_scale, "standard", (17, 13)) > 1e-4
