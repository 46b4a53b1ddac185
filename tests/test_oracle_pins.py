"""The oracle against facts other than itself (CPU only)."""

from __future__ import annotations

import math
import os

import numpy as np
import pytest

import oracle.muon_oracle as O
import workloads as W
from oracle_pins import (COEFFS, brute_force_index_map, gaussian_wide,
                         momentum_closed_form_error, quintic, runs_to_index_map,
                         svd_closed_form_error)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

WIDE_SHAPES = [(13, 17), (9, 17), (5, 5), (1, 7), (16, 64), (32, 33), (3, 200)]


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        line = [ln for ln in f if ln.strip() and not ln.startswith("#")][0]
    return dict(kv.split("=") for kv in line.split())


# ------------------------------------------------------------- NS closed form


@pytest.mark.parametrize("shape", WIDE_SHAPES)
@pytest.mark.parametrize("fn", [O.ns_standard, O.ns_gram], ids=["standard", "gram"])
def test_ns_matches_svd_closed_form(shape, fn):
    rng = np.random.default_rng(11 + shape[0] * 100 + shape[1])
    x = gaussian_wide(rng, *shape)
    assert svd_closed_form_error(fn, x) < 1e-12


@pytest.mark.parametrize("steps", [0, 1, 2, 3, 7])
def test_ns_step_count(steps):
    rng = np.random.default_rng(5)
    x = gaussian_wide(rng, 6, 11)
    for fn in (O.ns_standard, O.ns_gram):
        assert svd_closed_form_error(fn, x, steps=steps) < 1e-12


def test_quintic_worked_values():
    # f^k(1) for k = 1..5 of the scalar recurrence; f(1) = a + b + c exactly.
    a, b, c = COEFFS
    assert quintic(1.0, 1) == pytest.approx(a + b + c, abs=1e-15)
    seq = [float(quintic(1.0, k)) for k in range(1, 6)]
    assert seq[0] == pytest.approx(0.701, abs=1e-12)
    # A rank-1 input maps to f^5(1) times the outer product of its unit
    # singular vectors; f^5(1) lies in the contraction band below 1.
    assert 0.69 < seq[4] < 0.70


def test_rank1_input():
    p = np.array([1.0, -2.0, 0.5, 4.0])
    q = np.array([0.3, 0.1, -0.7, 2.0, 1.0, -1.0])
    g = np.outer(p, q)
    y = O.muon_matrix_update(g, "standard", eps=0.0)
    want = float(quintic(1.0)) * np.outer(p / np.linalg.norm(p), q / np.linalg.norm(q))
    assert np.max(np.abs(y - want)) < 1e-13


@pytest.mark.parametrize("m,n", [(2, 5), (4, 9), (13, 17), (128, 300)])
def test_orthonormal_rows(m, n):
    # Rows orthonormal => after normalisation every singular value is
    # 1/(sqrt(m) + eps), so the output is f^5 of that times the input rows.
    rng = np.random.default_rng(m * 7 + n)
    q, _ = np.linalg.qr(rng.standard_normal((n, m)))
    x = q.T  # m x n, orthonormal rows
    for method in ("standard", "gram"):
        y = O.muon_matrix_update(x, method)
        s = 1.0 / (math.sqrt(m) + O.NORM_EPS)
        assert np.max(np.abs(y - float(quintic(s)) * x)) < 1e-12


def test_output_singular_values_in_band():
    # For normalised inputs every singular value lies in (0, 1]; f^5 maps the
    # part of that interval above 1.5e-3 into [0.68, max f^5].
    grid = np.linspace(1.5e-3, 1.0, 200001)
    lo, hi = float(quintic(grid).min()), float(quintic(np.linspace(1e-6, 1.0, 200001)).max())
    assert 0.679 < lo and hi < 1.21
    for shape in [(17, 13), (9, 17), (64, 256)]:
        g = W.gaussian(shape, 3, 1.0).astype(np.float64)
        y = O.muon_matrix_update(g, "standard")
        s = np.linalg.svd(y, compute_uv=False)
        assert s.min() >= lo - 1e-9 and s.max() <= hi + 1e-9


# ----------------------------------------------------------------- forms


@pytest.mark.parametrize("shape", [(13, 17), (17, 13), (8, 8), (32, 32), (20, 90)])
def test_gram_equals_standard(shape):
    g = W.gaussian(shape, 42, 1.0).astype(np.float64)
    y1 = O.muon_matrix_update(g, "standard")
    y2 = O.muon_matrix_update(g, "gram")
    assert O.rel_frobenius(y2, y1) < 1e-12


def test_scale_invariance():
    g = W.gaussian((9, 17), 7, 1.0).astype(np.float64)
    base = O.muon_matrix_update(g, "standard", eps=0.0)
    for k in (-9, -1, 3, 20):
        np.testing.assert_array_equal(O.muon_matrix_update(g * 2.0 ** k, "standard", eps=0.0), base)
    for c in (0.37, 12.5, 1e-3):
        assert O.rel_frobenius(O.muon_matrix_update(g * c, "standard", eps=0.0), base) < 1e-13


def test_transpose_invariance():
    for shape in [(9, 17), (17, 13), (5, 40)]:
        g = W.gaussian(shape, 9, 1.0).astype(np.float64)
        for method in ("standard", "gram"):
            a = O.muon_matrix_update(g, method)
            b = O.muon_matrix_update(np.ascontiguousarray(g.T), method)
            np.testing.assert_array_equal(a, b.T)
    g = W.gaussian((12, 12), 9, 1.0).astype(np.float64)
    a = O.muon_matrix_update(g, "standard")
    b = O.muon_matrix_update(np.ascontiguousarray(g.T), "standard")
    assert O.rel_frobenius(b.T, a) < 1e-12


def test_zero_gradient_gives_zero_update():
    z = np.zeros((9, 17))
    for method in ("standard", "gram"):
        y = O.muon_matrix_update(z, method)
        assert np.all(y == 0.0) and np.all(np.isfinite(y))


# ----------------------------------------------------------------- per head


def test_per_head_one_head_is_unsplit():
    g = W.gaussian((16, 24), 1, 1.0).astype(np.float64)
    for h in (None, 0, 1):
        np.testing.assert_array_equal(O.muon_matrix_update(g, "standard", h),
                                      O.muon_matrix_update(g, "standard"))


@pytest.mark.parametrize("shape,h", [((16, 24), 2), ((12, 4), 2), ((32, 8), 4), ((128, 64), 8)])
def test_per_head_blocks_are_row_blocks(shape, h):
    g = W.gaussian(shape, 2, 1.0).astype(np.float64)
    y = O.muon_matrix_update(g, "standard", h)
    hr = shape[0] // h
    for b in range(h):
        blk = g[b * hr:(b + 1) * hr]
        np.testing.assert_array_equal(y[b * hr:(b + 1) * hr], O.muon_matrix_update(blk, "standard"))
        # closed form per block, independent of the oracle's block code
        x = blk.T if blk.shape[0] > blk.shape[1] else blk
        x = x / (np.linalg.norm(x) + O.NORM_EPS)
        U, S, Vt = np.linalg.svd(x, full_matrices=False)
        want = (U * quintic(S)) @ Vt
        want = want.T if blk.shape[0] > blk.shape[1] else want
        assert np.max(np.abs(y[b * hr:(b + 1) * hr] - want)) < 1e-12


def test_per_head_locality():
    g = W.gaussian((16, 24), 3, 1.0).astype(np.float64)
    y = O.muon_matrix_update(g, "gram", 4)
    g2 = g.copy()
    g2[12:16] *= -3.0
    g2[12, 0] += 1.0
    y2 = O.muon_matrix_update(g2, "gram", 4)
    np.testing.assert_array_equal(y[:12], y2[:12])
    assert not np.array_equal(y[12:], y2[12:])


def test_per_head_rejects_non_divisor():
    with pytest.raises(ValueError):
        O.muon_matrix_update(np.ones((10, 4)), "standard", 3)


# ------------------------------------------------------------- shape scale


def test_shape_scale():
    assert O.shape_scale(13, 17) == 1.0
    assert O.shape_scale(4096, 4096) == 1.0
    assert O.shape_scale(4096, 1024) == 2.0
    assert O.shape_scale(8192, 1024) == float(np.float32(2.0 * math.sqrt(2.0)))
    s = O.shape_scale(17, 13)
    assert s == float(np.float32(s))
    # the nearest fp32 to sqrt(17/13): its square brackets 17/13 within 1 ulp
    up = float(np.nextafter(np.float32(s), np.float32(2)))
    dn = float(np.nextafter(np.float32(s), np.float32(0)))
    assert abs(s * s - 17 / 13) <= min(abs(up * up - 17 / 13), abs(dn * dn - 17 / 13))


# ------------------------------------------------------------- momentum


@pytest.mark.parametrize("nesterov", [True, False])
def test_momentum_closed_form(nesterov):
    assert momentum_closed_form_error(O.momentum_update, 0.95, 5, nesterov) < 1e-6


def test_momentum_first_steps_values():
    g = np.ones((1, 1))
    m = np.zeros((1, 1), dtype=np.float32)
    got = []
    for _ in range(3):
        m, u = O.momentum_update(m, g, 0.95, True)
        got.append(float(u[0, 0]))
    # 1 - 0.95^2, 1 - 0.95^3, 1 - 0.95^4
    assert got == pytest.approx([0.0975, 0.142625, 0.18549375], rel=1e-6)


def test_constant_gradient_gives_identical_updates():
    g = W.gaussian((9, 17), 4, 1.0).astype(np.float64)
    state = O.init_state([(9, 17)])
    ys = []
    for _ in range(3):
        r = O.muon_step([g], state, [(9, 17)], [0], [0], 1, 160, O.MuonOptions())
        ys.append(r.updates[0])
    assert O.rel_frobenius(ys[1], ys[0]) < 1e-6 and O.rel_frobenius(ys[2], ys[0]) < 1e-6


# ---------------------------------------------------------- accumulation


def test_accumulate_sums_in_order():
    mbs = [np.full((2, 3), float(k)) for k in range(1, 5)]
    np.testing.assert_array_equal(O.accumulate(mbs), np.full((2, 3), 10.0))
    with pytest.raises(ValueError):
        O.accumulate([])


def _run_group(shapes, gas, steps, method="standard"):
    state = O.init_state(shapes)
    offsets, P = O.pack_layout(shapes, 2)
    outs = []
    for s in range(steps):
        grads = []
        for i, sh in enumerate(shapes):
            mbs = [W.gaussian(sh, W.grad_seed(0, i, k, s), 1.0) for k in range(gas)]
            grads.append(O.accumulate(mbs))
        outs.append(O.muon_step(grads, state, shapes, [0] * len(shapes), offsets, 2, P,
                                O.MuonOptions(method=method)))
    return state, outs


def test_ns_call_count_golden():
    gold = _golden("ns_call_count.txt")
    mats, steps, gas = int(gold["matrices"]), int(gold["steps"]), int(gold["gas"])
    state, _ = _run_group([(17, 13), (9, 17)][:mats], gas, steps)
    assert state.ns_invocations == int(gold["per_step"])
    assert state.ns_invocations != int(gold["per_microbatch"])
    assert state.steps == steps


def test_accumulation_equals_one_step_on_summed_gradient():
    shapes = [(17, 13), (9, 17)]
    gas = 3
    state_a, outs_a = _run_group(shapes, gas, 2)
    # same total gradient handed over as one pre-summed micro-batch
    state_b = O.init_state(shapes)
    offsets, P = O.pack_layout(shapes, 2)
    for s in range(2):
        grads = [sum(W.gaussian(sh, W.grad_seed(0, i, k, s), 1.0).astype(np.float64)
                     for k in range(gas)) for i, sh in enumerate(shapes)]
        out = O.muon_step(grads, state_b, shapes, [0, 0], offsets, 2, P, O.MuonOptions())
        for i in range(2):
            np.testing.assert_array_equal(out.updates[i], outs_a[s].updates[i])
    for i in range(2):
        np.testing.assert_array_equal(state_a.momenta[i], state_b.momenta[i])


# ------------------------------------------------------------- layout


def test_pack_layout_tiny():
    gold = _golden("tiny_group.txt")
    shapes = [tuple(int(v) for v in s.split("x")) for s in gold["shapes"].split(",")]
    R = int(gold["partitions"])
    offsets, P = O.pack_layout(shapes, R, 16)
    assert offsets == [0, 221] and P == 192
    offsets, P = O.pack_layout(shapes, R, 16, interior_align=True)
    assert offsets == [0, 224] and P == 192


@pytest.mark.parametrize("seed", range(8))
def test_partition_runs_brute_force(seed):
    rng = np.random.default_rng(seed)
    P = int(rng.integers(1, 50))
    for _ in range(20):
        off = int(rng.integers(0, 200))
        numel = int(rng.integers(1, 150))
        runs = O.partition_runs(off, numel, P)
        assert runs_to_index_map(runs, numel) == brute_force_index_map(off, numel, P)


def test_scatter_leaves_padding_untouched():
    shapes = [(17, 13), (9, 17)]
    for interior in (False, True):
        offsets, P = O.pack_layout(shapes, 2, 16, interior_align=interior)
        sentinel = np.array([0x7FBADBAD], dtype=np.uint32).view(np.float32)[0]
        parts = [np.full(P, sentinel, dtype=np.float32) for _ in range(2)]
        covered = np.zeros(2 * P, dtype=bool)
        for (r, c), off in zip(shapes, offsets):
            val = np.arange(r * c, dtype=np.float32).reshape(r, c) + 1.0
            O.scatter_f32(val, off, parts)
            covered[off:off + r * c] = True
            np.testing.assert_array_equal(O.gather_from_partitions(parts, off, r, c), val)
        flat = np.concatenate(parts).view(np.uint32)
        assert np.all(flat[~covered] == 0x7FBADBAD)
        assert not np.any(flat[covered] == 0x7FBADBAD)


def test_scaled_update_is_one_fp32_multiply():
    y = W.gaussian((17, 13), 5, 1.0)
    got = O.scaled_update_f32(y, 17, 13)
    s = np.float32(O.shape_scale(17, 13))
    # each product rounded once from the exact product (fp64 holds it exactly)
    exact = y.astype(np.float64) * np.float64(s)
    np.testing.assert_array_equal(got, exact.astype(np.float32))


def test_step_writes_scaled_update():
    shapes = [(17, 13), (9, 17)]
    state, outs = _run_group(shapes, 3, 1)
    offsets, P = O.pack_layout(shapes, 2)
    for i, (r, c) in enumerate(shapes):
        got = O.gather_from_partitions(outs[0].partitions, offsets[i], r, c)
        want = outs[0].ns_out[i] * O.shape_scale(r, c)
        assert O.rel_frobenius(got, want) < 1e-7


# ------------------------------------------- loss scale and discarded steps


def test_grad_scale_momentum_closed_form():
    # one step from zero momentum: m = (1 - beta) * s * g exactly as fp32 of
    # the fp64 product (s a power of two keeps s * g exact)
    g = W.gaussian((9, 17), 21, 1.0).astype(np.float64)
    for s in (1.0, 2.0 ** -12, 8.0):
        state = O.init_state([(9, 17)])
        O.muon_step([g], state, [(9, 17)], [0], [0], 1, 160, O.MuonOptions(), grad_scale=s)
        np.testing.assert_array_equal(state.momenta[0], ((1.0 - 0.95) * s * g).astype(np.float32))


def test_grad_scale_cancels_loss_scale():
    # gradients produced under loss scale S, handed in with grad_scale 1/S,
    # give the unscaled run's momentum and updates (S a power of two: exact)
    shapes = [(17, 13), (9, 17)]
    offsets, P = O.pack_layout(shapes, 2)
    ref_state, sc_state = O.init_state(shapes), O.init_state(shapes)
    for step in range(2):
        grads = [W.gaussian(sh, W.grad_seed(0, i, 0, step), 1.0).astype(np.float64) for i, sh in enumerate(shapes)]
        a = O.muon_step(grads, ref_state, shapes, [0, 0], offsets, 2, P, O.MuonOptions())
        S = 2.0 ** (10 + step)
        b = O.muon_step([g * S for g in grads], sc_state, shapes, [0, 0], offsets, 2, P, O.MuonOptions(),
                        grad_scale=1.0 / S)
        for i in range(2):
            np.testing.assert_array_equal(sc_state.momenta[i], ref_state.momenta[i])
            np.testing.assert_array_equal(b.partitions[i], a.partitions[i])


def test_skipped_step_touches_nothing():
    shapes = [(17, 13), (9, 17)]
    offsets, P = O.pack_layout(shapes, 2)
    grads = [W.gaussian(sh, 70 + i, 1.0).astype(np.float64) for i, sh in enumerate(shapes)]
    state = O.init_state(shapes)
    O.muon_step(grads, state, shapes, [0, 0], offsets, 2, P, O.MuonOptions())
    mom = [m.copy() for m in state.momenta]
    parts = [np.full(P, 7.0, dtype=np.float32) for _ in range(2)]
    r = O.muon_step([g * np.inf for g in grads], state, shapes, [0, 0], offsets, 2, P, O.MuonOptions(),
                    partitions=parts, skip=True)
    assert state.steps == 1 and state.ns_invocations == 2
    for i in range(2):
        np.testing.assert_array_equal(state.momenta[i], mom[i])
        np.testing.assert_array_equal(r.partitions[i], np.full(P, 7.0, dtype=np.float32))
    # a run with the discarded step in between equals the run without it
    state2 = O.init_state(shapes)
    O.muon_step(grads, state2, shapes, [0, 0], offsets, 2, P, O.MuonOptions())
    g2 = [W.gaussian(sh, 90 + i, 1.0).astype(np.float64) for i, sh in enumerate(shapes)]
    ra = O.muon_step(g2, state, shapes, [0, 0], offsets, 2, P, O.MuonOptions())
    rb = O.muon_step(g2, state2, shapes, [0, 0], offsets, 2, P, O.MuonOptions())
    for i in range(2):
        np.testing.assert_array_equal(ra.partitions[i], rb.partitions[i])


# ----------------------------------------- update norm, clipping, param update


def _tiny_layout_with_values():
    # two matrices 1x2 and 2x2 in two partitions of 4: flat [0..6), padding at
    # flat 6 and 7 (partition 1, offsets 2 and 3)
    shapes, offsets, P = [(1, 2), (2, 2)], [0, 2], 4
    parts = [np.array([3.0, 4.0, 1.0, 2.0], dtype=np.float32),
             np.array([2.0, 4.0, np.nan, np.nan], dtype=np.float32)]
    return shapes, offsets, P, parts


def test_update_norm_hand_values():
    shapes, offsets, P, parts = _tiny_layout_with_values()
    # 9 + 16 + 1 + 4 + 4 + 16 = 50; padding (NaN) excluded
    assert O.update_norm(parts, shapes, offsets) == pytest.approx(math.sqrt(50.0), abs=1e-15)


def test_update_norm_equals_per_matrix_sum():
    shapes = [(17, 13), (9, 17), (5, 40)]
    state, outs = _run_group(shapes, 1, 1)
    offsets, P = O.pack_layout(shapes, 2)
    parts = outs[0].partitions
    per = sum(float(np.sum(O.gather_from_partitions(parts, offsets[i], r, c).astype(np.float64) ** 2))
              for i, (r, c) in enumerate(shapes))
    assert O.update_norm(parts, shapes, offsets) == pytest.approx(math.sqrt(per), rel=1e-14)


def test_clip_coefficient_cases():
    assert O.clip_coefficient(10.0, 0.0) == 1.0
    assert O.clip_coefficient(10.0, -1.0) == 1.0
    assert O.clip_coefficient(0.5, 1.0) == 1.0
    assert O.clip_coefficient(10.0, 1.0) == pytest.approx(1.0 / (10.0 + 1e-6), rel=1e-15)
    assert O.clip_coefficient(0.0, 1.0) == 1.0


def test_apply_update_closed_forms():
    shapes, offsets, P, parts = _tiny_layout_with_values()
    params = [np.array([1.0, -1.0, 0.5, 2.0], dtype=np.float32),
              np.array([0.25, 8.0, 5.0, -5.0], dtype=np.float32)]
    # lr = 0: nothing moves
    out, norm, clip = O.apply_update(params, parts, shapes, offsets, 0.0, 0.1, 0.0)
    for a, b in zip(out, params):
        np.testing.assert_array_equal(a, b)
    # no decay, no clipping: p - lr * u, exact for these values (lr 1/4)
    out, norm, clip = O.apply_update(params, parts, shapes, offsets, 0.25, 0.0, 0.0)
    assert clip == 1.0 and norm == pytest.approx(math.sqrt(50.0))
    np.testing.assert_array_equal(out[0], np.array([0.25, -2.0, 0.25, 1.5], dtype=np.float32))
    np.testing.assert_array_equal(out[1][:2], np.array([-0.25, 7.0], dtype=np.float32))
    # padding untouched (the update there is NaN, the params keep their values)
    np.testing.assert_array_equal(out[1][2:], params[1][2:])
    # decay only: zero update
    zero = [np.zeros(4, dtype=np.float32), np.zeros(4, dtype=np.float32)]
    out, _, _ = O.apply_update(params, zero, shapes, offsets, 0.5, 0.5, 0.0)
    np.testing.assert_array_equal(out[0], (params[0] * 0.75).astype(np.float32))
    # skipped step: unchanged
    out, _, _ = O.apply_update(params, parts, shapes, offsets, 0.25, 0.1, 1.0, skip=True)
    for a, b in zip(out, params):
        np.testing.assert_array_equal(a, b)


def test_apply_update_clipped_step_has_max_norm():
    shapes = [(17, 13), (9, 17)]
    state, outs = _run_group(shapes, 1, 1)
    offsets, P = O.pack_layout(shapes, 2)
    parts = outs[0].partitions
    params = [np.zeros(P, dtype=np.float32) for _ in range(2)]
    lr, max_norm = 0.5, 0.125
    out, norm, clip = O.apply_update(params, parts, shapes, offsets, lr, 0.0, max_norm)
    assert norm > max_norm and clip < 1.0
    step = [-(o.astype(np.float64)) for o in out]
    total = math.sqrt(sum(float(np.dot(s, s)) for s in step))
    assert total == pytest.approx(lr * max_norm * norm / (norm + 1e-6), rel=1e-6)


# ------------------------------------------------------ decoding and metric


def test_bf16_decode_known_patterns():
    from oracle_pins import bf16_decode_error
    assert bf16_decode_error(O.bf16_bits_to_f64) == 0
    assert bf16_decode_error(lambda b: O.as_f64(b, "bf16")) == 0


def test_as_f64_fp32_is_exact_widening():
    x = np.array([1.0, -0.1, 3.4028234663852886e38, 1.401298464324817e-45, -0.0], dtype=np.float32)
    got = O.as_f64(x, "fp32")
    assert got.dtype == np.float64
    # every fp32 value is an fp64 value: widening changes no bit of the value
    np.testing.assert_array_equal(got.astype(np.float32).view(np.uint32), x.view(np.uint32))
    assert got[1] == float(np.float32(-0.1)) and got[1] != -0.1
    with pytest.raises(ValueError):
        O.as_f64(x, "fp16")


def test_rel_frobenius_hand_values():
    # ||got - want|| / ||want||, not divided by ||got||
    assert O.rel_frobenius([1.0, 0.0], [0.0, 2.0]) == pytest.approx(math.sqrt(5.0) / 2.0, rel=1e-15)
    assert O.rel_frobenius([0.0, 2.0], [1.0, 0.0]) == pytest.approx(math.sqrt(5.0), rel=1e-15)
    # a 3-4-5 difference over a norm-10 reference
    assert O.rel_frobenius([[6.0, 8.0], [0.0, 0.0]], [[3.0, 4.0], [0.0, 0.0]]) == pytest.approx(1.0, rel=1e-15)
    assert O.rel_frobenius([[9.0, 4.0]], [[6.0, 8.0]]) == pytest.approx(0.5, rel=1e-15)
    # equal inputs, and the 0/0 and x/0 branches
    assert O.rel_frobenius([1.5, -2.0], [1.5, -2.0]) == 0.0
    assert O.rel_frobenius([0.0, 0.0], [0.0, 0.0]) == 0.0
    assert O.rel_frobenius([0.0, 1e-30], [0.0, 0.0]) == math.inf
    # sign and scale: -want is at distance 2, 2*want at distance 1
    w = W.gaussian((7, 5), 3, 1.0)
    assert O.rel_frobenius(-w, w) == pytest.approx(2.0, rel=1e-14)
    assert O.rel_frobenius(2.0 * w, w) == pytest.approx(1.0, rel=1e-14)


def test_gather_from_partitions_brute_force():
    # partition r, offset o holds the value of its flat index r*P + o, so
    # reading a matrix back must give flat_offset + j at element j
    P, R = 13, 4
    parts = [np.arange(r * P, (r + 1) * P, dtype=np.float32) for r in range(R)]
    for off, (rows, cols) in ((0, (3, 4)), (5, (2, 9)), (11, (5, 7)), (38, (1, 14))):
        got = O.gather_from_partitions(parts, off, rows, cols)
        np.testing.assert_array_equal(got, (off + np.arange(rows * cols, dtype=np.float32)).reshape(rows, cols))


# ------------------------------------- the whole step with a warm momentum


@pytest.mark.parametrize("shape", [(9, 17), (17, 13), (12, 12)])
@pytest.mark.parametrize("method", ["standard", "gram"])
def test_step_nesterov_blend_closed_form(method, shape):
    from oracle_pins import nesterov_step_error
    assert nesterov_step_error(O.muon_step, method, shape) < 1e-12
