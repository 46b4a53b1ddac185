"""HIP path vs the oracle, element by element on the same seeded inputs.

Tolerances (per matrix, relative Frobenius error of the scaled update against
the fp64 oracle): 1e-4 on the fp32 Newton-Schulz path and 2e-2 on the bf16
MFMA path.  The writeback is bit-exact and padding untouched.  Momentum is
within 3 fp32 spacings of the magnitude of its terms beta*m and (1-beta)*g
(the evaluation error of a two-term fp32 expression; counting raw ulps of
the result is meaningless where the two terms cancel).  Every case runs
through the C ABI on cuda:0.
"""

from __future__ import annotations

import numpy as np
import pytest

import muon_newton_schulz_step_amd as M
import oracle.muon_oracle as O
import workloads as W
from gpu_util import SENTINEL, assert_tiles_within, host, run_steps, sentinel_partitions, to_device, workspace

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.load()
    yield


def _oracle_run(shapes, heads, offsets, R, P, micro, micro_dtype, method, steps_ns=5, nesterov=True,
                momenta0=None, beta=0.95, coeffs=O.NS_COEFFS):
    """Run the oracle over the same micro-batches.  Also returns, per matrix,
    the largest |beta m_prev| + |(1-beta) g| seen over the steps: the scale of
    the terms whose fp32 evaluation the momentum check bounds."""
    state = O.init_state(shapes)
    if momenta0 is not None:
        state.momenta = [m.astype(np.float32).copy() for m in momenta0]
    b = float(np.float32(beta))
    opt = O.MuonOptions(beta=b, nesterov=nesterov, method=method, steps=steps_ns, coeffs=coeffs,
                        eps=float(np.float32(O.NORM_EPS)))
    res = None
    sentinel = np.array([SENTINEL], dtype=np.uint32).view(np.float32)[0]
    parts = [np.full(P, sentinel, dtype=np.float32) for _ in range(R)]
    mag = [np.zeros(s) for s in shapes]
    for step in micro:
        grads = [O.accumulate([O.as_f64(mb[i], micro_dtype) for mb in step]) for i in range(len(shapes))]
        for i in range(len(shapes)):
            mag[i] = np.maximum(mag[i], np.abs(b * state.momenta[i].astype(np.float64)) + np.abs((1 - b) * grads[i]))
        res = O.muon_step(grads, state, shapes, heads, offsets, R, P, opt, partitions=parts)
    res.term_scale = mag
    return res, state


def _check_momentum(moms_gpu, state, res, ulps=3):
    """fp32 momentum vs the oracle's (fp64, rounded once): within a few fp32
    spacings of the magnitude of the terms beta*m and (1-beta)*g."""
    for i, (got, want) in enumerate(zip(moms_gpu, state.momenta)):
        bound = ulps * np.spacing(res.term_scale[i].astype(np.float32)).astype(np.float64)
        diff = np.abs(got.astype(np.float64) - want.astype(np.float64))
        assert np.all(diff <= bound), f"momentum {i}: worst {np.max(diff / np.maximum(bound, 1e-45)):.2f} x bound"


def _compare(shapes, offsets, parts_gpu, res, tol, label=""):
    """Per matrix, and per 256 x 256 block of it (the last blocks being the
    ragged edge strips), relative Frobenius error within tol: a wrong tile or
    edge strip of a large matrix cannot hide in the matrix-level figure."""
    worst = 0.0
    for i, (r, c) in enumerate(shapes):
        got = O.gather_from_partitions(parts_gpu, offsets[i], r, c)
        err = O.rel_frobenius(got, res.updates[i])
        worst = max(worst, err)
        assert err <= tol, f"{label} matrix {i} {r}x{c}: rel err {err:.3e} > {tol}"
        assert_tiles_within(got, res.updates[i], tol, f"{label} matrix {i} {r}x{c}")
    return worst


def _check_padding(parts_gpu, shapes, offsets, P):
    flat = np.concatenate(parts_gpu).view(np.uint32)
    covered = np.zeros(flat.size, dtype=bool)
    for (r, c), off in zip(shapes, offsets):
        covered[off:off + r * c] = True
    assert np.all(flat[~covered] == SENTINEL), "padding was written"
    assert not np.any(flat[covered] == SENTINEL)


def _micro(shapes, dtype, sigma, gas, steps, cid=7):
    return [[[W.make_grad(s, W.grad_seed(cid, i, k, t), sigma, dtype) for i, s in enumerate(shapes)]
             for k in range(gas)] for t in range(steps)]


# ------------------------------------------------------------------ tiny


@pytest.mark.parametrize("method", ["standard", "gram"])
@pytest.mark.parametrize("interior", [False, True])
def test_tiny_group_fp32(method, interior):
    wl = W.tiny()
    offsets, P = O.pack_layout(wl.shapes, wl.num_partitions, 16, interior_align=interior)
    g = M.MuonGroup(wl.shapes, offsets=offsets, num_partitions=2, partition_numel=P, method=method,
                    precision="fp32", grad_dtype="fp32")
    micro = _micro(wl.shapes, "fp32", 1.0, wl.gas, wl.steps, cid=0)
    parts, moms = run_steps(g, micro, "fp32")
    res, state = _oracle_run(wl.shapes, wl.heads, offsets, 2, P, micro, "fp32", method)
    _compare(wl.shapes, offsets, parts, res, TOL["fp32"], f"tiny/{method}")
    _check_padding(parts, wl.shapes, offsets, P)
    _check_momentum(moms, state, res)
    st = g.stats()
    assert st["steps"] == 3 and st["ns_invocations"] == 2 * 3 and st["accumulations"] == 9


@pytest.mark.parametrize("method", ["standard", "gram"])
def test_tiny_group_bf16_precision(method):
    # Blocks with fewer than 64 rows run on fp32 operands even on the bf16
    # path, so these small matrices meet the fp32 bar.
    wl = W.tiny()
    offsets, P = O.pack_layout(wl.shapes, 2, 16)
    g = M.MuonGroup(wl.shapes, offsets=offsets, num_partitions=2, partition_numel=P, method=method,
                    precision="bf16", grad_dtype="fp32")
    micro = _micro(wl.shapes, "fp32", 1.0, wl.gas, wl.steps, cid=0)
    parts, _ = run_steps(g, micro, "fp32")
    res, _ = _oracle_run(wl.shapes, wl.heads, offsets, 2, P, micro, "fp32", method)
    worst = _compare(wl.shapes, offsets, parts, res, TOL["fp32"], f"tiny-bf16/{method}")
    print(f"tiny bf16 {method}: worst rel err {worst:.3e}")
    _check_padding(parts, wl.shapes, offsets, P)


# --------------------------------------------------- several tiles, ragged

MID_SHAPES = [(300, 200), (130, 520), (257, 257), (256, 512), (512, 64), (96, 640), (1, 33), (40, 1)]
MID_HEADS = [0, 0, 0, 4, 2, 3, 0, 0]


@pytest.mark.parametrize("precision", ["fp32", "bf16"])
@pytest.mark.parametrize("method", ["standard", "gram"])
def test_mid_group(precision, method):
    offsets, P = O.pack_layout(MID_SHAPES, 3, 16, interior_align=True)
    g = M.MuonGroup(MID_SHAPES, heads=MID_HEADS, offsets=offsets, num_partitions=3, partition_numel=P,
                    method=method, precision=precision, grad_dtype="bf16")
    micro = _micro(MID_SHAPES, "bf16", 0.02, 1, 2, cid=11)
    m0 = [W.warm_momentum(s, 77 + i, 0.02) for i, s in enumerate(MID_SHAPES)]
    parts, moms = run_steps(g, micro, "bf16", momenta0=m0, use_accumulate=False)
    res, state = _oracle_run(MID_SHAPES, MID_HEADS, offsets, 3, P, micro, "bf16", method, momenta0=m0)
    worst = _compare(MID_SHAPES, offsets, parts, res, TOL[precision], f"mid/{precision}/{method}")
    print(f"mid {precision} {method}: worst rel err {worst:.3e}")
    _check_padding(parts, MID_SHAPES, offsets, P)
    _check_momentum(moms, state, res)


@pytest.mark.parametrize("precision", ["fp32", "bf16"])
@pytest.mark.parametrize("steps_ns", [0, 1, 2, 3])
@pytest.mark.parametrize("method", ["standard", "gram"])
def test_ns_step_counts(steps_ns, method, precision):
    shapes = [(70, 150), (150, 70), (128, 128)]
    offsets, P = O.pack_layout(shapes, 1, 16)
    g = M.MuonGroup(shapes, method=method, precision=precision, grad_dtype="fp32", ns_steps=steps_ns)
    micro = _micro(shapes, "fp32", 1.0, 1, 1, cid=12)
    parts, _ = run_steps(g, micro, "fp32", use_accumulate=False)
    res, _ = _oracle_run(shapes, [0, 0, 0], offsets, 1, P, micro, "fp32", method, steps_ns=steps_ns)
    _compare(shapes, offsets, parts, res, TOL[precision], f"T={steps_ns}/{method}/{precision}")


@pytest.mark.parametrize("precision", ["fp32", "bf16"])
@pytest.mark.parametrize("method", ["standard", "gram"])
def test_custom_coefficients_and_step_count(method, precision):
    # (a, b, c) and the step count come from the options: the quintic
    # 2x - 1.5x^3 + 0.5x^5 over 7 steps, on every kernel kind (a large-tile
    # block, two fused ones, an fp32-operand one)
    shapes = [(300, 520), (128, 700), (96, 96), (40, 90)]
    coeffs = (2.0, -1.5, 0.5)
    offsets, P = O.pack_layout(shapes, 1, 16)
    g = M.MuonGroup(shapes, method=method, precision=precision, grad_dtype="fp32", ns_steps=7, coeffs=coeffs)
    micro = _micro(shapes, "fp32", 1.0, 1, 1, cid=13)
    parts, _ = run_steps(g, micro, "fp32", use_accumulate=False)
    res, _ = _oracle_run(shapes, [0] * len(shapes), offsets, 1, P, micro, "fp32", method, steps_ns=7,
                         coeffs=coeffs)
    _compare(shapes, offsets, parts, res, TOL[precision], f"coeffs/{method}/{precision}")


def test_nesterov_off_and_beta():
    shapes = [(64, 96), (96, 64)]
    offsets, P = O.pack_layout(shapes, 1, 16)
    g = M.MuonGroup(shapes, precision="fp32", grad_dtype="fp32", nesterov=False, beta=0.9)
    micro = _micro(shapes, "fp32", 1.0, 1, 2, cid=13)
    m0 = [W.warm_momentum(s, 5, 1.0) for s in shapes]
    parts, moms = run_steps(g, micro, "fp32", momenta0=m0, use_accumulate=False)
    res, state = _oracle_run(shapes, [0, 0], offsets, 1, P, micro, "fp32", "standard", nesterov=False,
                             momenta0=m0, beta=0.9)
    _compare(shapes, offsets, parts, res, TOL["fp32"], "nesterov-off")
    _check_momentum(moms, state, res)


DEGEN_SHAPES = [(1, 1), (1, 2), (2, 1), (3, 3), (1, 300), (257, 1)]


@pytest.mark.parametrize("precision", ["fp32", "bf16"])
@pytest.mark.parametrize("method", ["standard", "gram"])
def test_degenerate_shapes_and_beta_zero(precision, method):
    # single elements, single rows and columns (rank-one blocks, 1 x 1
    # Newton-Schulz problems) crossing two partitions, with beta = 0 so the
    # momentum is the gradient itself
    offsets, P = O.pack_layout(DEGEN_SHAPES, 2, 16)
    g = M.MuonGroup(DEGEN_SHAPES, offsets=offsets, num_partitions=2, partition_numel=P, method=method,
                    precision=precision, grad_dtype="fp32", beta=0.0)
    micro = _micro(DEGEN_SHAPES, "fp32", 1.0, 1, 2, cid=51)
    parts, moms = run_steps(g, micro, "fp32", use_accumulate=False)
    res, state = _oracle_run(DEGEN_SHAPES, [0] * len(DEGEN_SHAPES), offsets, 2, P, micro, "fp32", method, beta=0.0)
    _compare(DEGEN_SHAPES, offsets, parts, res, TOL[precision], f"degenerate/{method}/{precision}")
    _check_padding(parts, DEGEN_SHAPES, offsets, P)
    _check_momentum(moms, state, res)
    # beta = 0: the momentum after the last step is that step's gradient
    for i, m in enumerate(moms):
        np.testing.assert_array_equal(m, micro[-1][0][i])


def test_zero_gradient_zero_update():
    shapes = [(33, 65), (65, 33)]
    g = M.MuonGroup(shapes, precision="bf16", grad_dtype="fp32")
    micro = [[[np.zeros(s, dtype=np.float32) for s in shapes]]]
    parts, moms = run_steps(g, micro, "fp32", use_accumulate=False)
    flat = np.concatenate(parts)[:sum(r * c for r, c in shapes)]
    assert np.all(flat == 0.0)
    assert all(np.all(m == 0.0) for m in moms)


# ----------------------------------------------------------- writeback


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_scatter_bit_exact(dtype):
    torch = pytest.importorskip("torch")
    shapes = [(17, 13), (9, 17), (100, 37), (5, 300)]
    for R, interior in ((1, False), (2, False), (3, True), (7, True)):
        offsets, P = O.pack_layout(shapes, R, 16, interior_align=interior)
        g = M.MuonGroup(shapes, offsets=offsets, num_partitions=R, partition_numel=P)
        ups_host = [W.make_grad(s, 900 + i, 1.0, dtype) for i, s in enumerate(shapes)]
        ups = [to_device(u, dtype) for u in ups_host]
        parts = sentinel_partitions(R, P)
        ws_t, ws = workspace(g.workspace_bytes)
        g.scatter(ups, dtype, parts, ws)
        torch.cuda.synchronize()
        got = [host(p) for p in parts]
        sentinel = np.array([SENTINEL], dtype=np.uint32).view(np.float32)[0]
        want = [np.full(P, sentinel, dtype=np.float32) for _ in range(R)]
        for i, (r, c) in enumerate(shapes):
            val = O.as_f64(ups_host[i], dtype).astype(np.float32).reshape(r, c)
            O.scatter_f32(O.scaled_update_f32(val, r, c), offsets[i], want)
        np.testing.assert_array_equal(np.concatenate(got).view(np.uint32), np.concatenate(want).view(np.uint32))


def test_accumulate_bit_exact_fp32_sequence():
    torch = pytest.importorskip("torch")
    shapes = [(37, 41), (8, 1000)]
    g = M.MuonGroup(shapes, grad_dtype="fp32")
    ws_t, ws = workspace(g.workspace_bytes)
    accs = [torch.empty(r, c, dtype=torch.float32, device="cuda:0") for r, c in shapes]
    for dtype in ("bf16", "fp32"):
        mbs = [[W.make_grad(s, 300 + 10 * k + i, 1.0, dtype) for i, s in enumerate(shapes)] for k in range(4)]
        for k, mb in enumerate(mbs):
            g.accumulate(accs, [to_device(x, dtype) for x in mb], dtype, k == 0, ws)
            torch.cuda.synchronize()
        for i in range(len(shapes)):
            want = O.as_f64(mbs[0][i], dtype).astype(np.float32)
            for k in range(1, 4):
                want = (want + O.as_f64(mbs[k][i], dtype).astype(np.float32)).astype(np.float32)
            np.testing.assert_array_equal(host(accs[i]), want)


@pytest.mark.parametrize("method", ["standard", "gram"])
def test_deterministic_and_wave_invariant(method):
    # 128-tile, fused (128 x 128) and large-tile-free blocks; run twice and in
    # one wave per matrix: the same bits
    shapes = [(200, 300), (300, 200), (128, 128), (64, 512)]
    micro = _micro(shapes, "bf16", 0.02, 1, 1, cid=21)
    outs = []
    for cap in (0, 0, 1):
        g = M.MuonGroup(shapes, heads=[0, 0, 0, 2], precision="bf16", grad_dtype="bf16", method=method,
                        max_inflight_bytes=cap)
        if cap:
            assert g.stats()["waves"] == len(shapes)
        parts, moms = run_steps(g, micro, "bf16", use_accumulate=False)
        outs.append((np.concatenate(parts).view(np.uint32), [m.view(np.uint32) for m in moms]))
    for o in outs[1:]:
        np.testing.assert_array_equal(o[0], outs[0][0])
        for a, b in zip(o[1], outs[0][1]):
            np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("method,cap", [("standard", 4 << 20), ("gram", 6 << 20)])
def test_mixed_sizes_waves_and_second_stream_bitwise(method, cap):
    # large-tile problems (m >= 256) beside small-block ones (head blocks,
    # m < 256, fp32-operand blocks): the small groups run on the plan's
    # second stream, joined before the writeback.  Capped, the group runs in
    # three workspace waves, two of which hold both kinds (a fork and a join
    # per wave); one wave and three give the same bits, and the one-wave run
    # matches the oracle.
    shapes = [(512, 700), (300, 200), (260, 300), (1024, 256), (600, 280), (64, 900), (33, 65)]
    heads = [0, 0, 0, 8, 0, 0, 0]
    offsets, P = O.pack_layout(shapes, 2, 16)
    micro = _micro(shapes, "bf16", 0.02, 1, 2, cid=61)
    outs = []
    for c in (0, cap):
        g = M.MuonGroup(shapes, heads=heads, offsets=offsets, num_partitions=2, partition_numel=P, method=method,
                        precision="bf16", grad_dtype="bf16", max_inflight_bytes=c)
        waves = {}
        for q in g.problems():
            waves.setdefault(q["wave"], set()).add(q["m"] >= 256)
        assert len(waves) == (1 if c == 0 else 3)
        assert sum(1 for kinds in waves.values() if len(kinds) == 2) == (1 if c == 0 else 2)
        parts, moms = run_steps(g, micro, "bf16", use_accumulate=False)
        outs.append((parts, moms))
    for a, b in zip(outs[0][0] + outs[0][1], outs[1][0] + outs[1][1]):
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
    res, state = _oracle_run(shapes, heads, offsets, 2, P, micro, "bf16", method)
    _compare(shapes, offsets, outs[0][0], res, TOL["bf16"], f"mixed/{method}")
    _check_padding(outs[0][0], shapes, offsets, P)
    _check_momentum(outs[0][1], state, res)


def test_per_head_toggle_changes_only_tagged():
    shapes = [(256, 128), (128, 384)]
    micro = _micro(shapes, "bf16", 0.02, 1, 1, cid=31)
    a = M.MuonGroup(shapes, heads=[0, 0], precision="fp32", grad_dtype="bf16")
    b = M.MuonGroup(shapes, heads=[4, 0], precision="fp32", grad_dtype="bf16")
    pa, _ = run_steps(a, micro, "bf16", use_accumulate=False)
    pb, _ = run_steps(b, micro, "bf16", use_accumulate=False)
    fa, fb = np.concatenate(pa), np.concatenate(pb)
    n0 = 256 * 128
    assert not np.array_equal(fa[:n0], fb[:n0])
    np.testing.assert_array_equal(fa[n0:n0 + 128 * 384].view(np.uint32), fb[n0:n0 + 128 * 384].view(np.uint32))


# --------------------------------------------- large-tile kernel (m >= 256)

BIG_SHAPES = [(512, 700), (700, 300), (256, 256), (600, 1100), (1024, 512)]


@pytest.mark.parametrize("method", ["standard", "gram"])
def test_big_tile_group(method):
    # small sides 256..600 with ragged M/N/K against the 256-wide tiles and
    # the 64-deep K stages (700 = 10*64 + 60, 1100 = 17*64 + 12)
    offsets, P = O.pack_layout(BIG_SHAPES, 2, 16)
    g = M.MuonGroup(BIG_SHAPES, offsets=offsets, num_partitions=2, partition_numel=P, method=method,
                    precision="bf16", grad_dtype="bf16")
    micro = _micro(BIG_SHAPES, "bf16", 0.02, 1, 1, cid=41)
    parts, moms = run_steps(g, micro, "bf16", use_accumulate=False)
    res, state = _oracle_run(BIG_SHAPES, [0] * len(BIG_SHAPES), offsets, 2, P, micro, "bf16", method)
    worst = _compare(BIG_SHAPES, offsets, parts, res, TOL["bf16"], f"big/{method}")
    print(f"big-tile bf16 {method}: worst rel err {worst:.3e}")
    _check_padding(parts, BIG_SHAPES, offsets, P)
    _check_momentum(moms, state, res)


LEAN_SHAPES = [(2048, 2048), (2304, 2112), (3000, 2080), (1024, 1100)]


def test_gram_lean_q_chain():
    # Gram blocks with m >= 2048 accumulate Q with one bf16 product: a square
    # block, a wide and a tall one ragged against the 256 tiles (m = 2112,
    # 2080), beside a 1024-row block on the full split chain
    offsets, P = O.pack_layout(LEAN_SHAPES, 2, 16)
    g = M.MuonGroup(LEAN_SHAPES, offsets=offsets, num_partitions=2, partition_numel=P, method="gram",
                    precision="bf16", grad_dtype="bf16")
    assert [q["m"] for q in g.problems()] == [2048, 2112, 2080, 1024]
    micro = _micro(LEAN_SHAPES, "bf16", 0.02, 1, 1, cid=45)
    parts, moms = run_steps(g, micro, "bf16", use_accumulate=False)
    res, state = _oracle_run(LEAN_SHAPES, [0] * len(LEAN_SHAPES), offsets, 2, P, micro, "bf16", "gram")
    worst = _compare(LEAN_SHAPES, offsets, parts, res, TOL["bf16"], "gram-lean")
    print(f"gram lean Q chain: worst rel err {worst:.3e}")
    _check_padding(parts, LEAN_SHAPES, offsets, P)


BIG_HEAD_SHAPES = [(1024, 600), (768, 300), (1200, 256)]
BIG_HEAD_COUNTS = [2, 3, 2]


@pytest.mark.parametrize("method", ["standard", "gram"])
def test_big_tile_head_blocks(method):
    # head blocks on the large-tile kernel: 512 x 600 (two per matrix),
    # 256 x 300 (three, ragged K) and 600 x 256 (two tall blocks, stored
    # transposed), each block its own Newton-Schulz problem in the workspace
    offsets, P = O.pack_layout(BIG_HEAD_SHAPES, 2, 16)
    g = M.MuonGroup(BIG_HEAD_SHAPES, heads=BIG_HEAD_COUNTS, offsets=offsets, num_partitions=2, partition_numel=P,
                    method=method, precision="bf16", grad_dtype="bf16")
    probs = g.problems()
    assert [(q["m"], q["n"], q["transposed"]) for q in probs] == \
        [(512, 600, False)] * 2 + [(256, 300, False)] * 3 + [(256, 600, True)] * 2
    micro = _micro(BIG_HEAD_SHAPES, "bf16", 0.02, 1, 1, cid=43)
    parts, moms = run_steps(g, micro, "bf16", use_accumulate=False)
    res, state = _oracle_run(BIG_HEAD_SHAPES, BIG_HEAD_COUNTS, offsets, 2, P, micro, "bf16", method)
    worst = _compare(BIG_HEAD_SHAPES, offsets, parts, res, TOL["bf16"], f"big-heads/{method}")
    print(f"big-tile head blocks bf16 {method}: worst rel err {worst:.3e}")
    _check_padding(parts, BIG_HEAD_SHAPES, offsets, P)
    _check_momentum(moms, state, res)
