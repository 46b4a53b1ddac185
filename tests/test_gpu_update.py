"""The inputs a training loop adds around the step, on the GPU through the C
ABI: the gradient scale, the device-side skip flag of a discarded step, the
overflow check that produces it, the norm / clip / parameter update after the
step, and an interrupted-vs-uninterrupted checkpoint run.

Tolerances: the gradient scale and the skip flag are checked bit for bit
against the plain step (a power-of-two scale is exact).  The update norm
against the oracle's fp64 norm of the same partitions: 1e-6 relative (fp32
partial sums of 4096 squares).  Parameters: within 2 fp32 spacings of the
larger of |p (1 - lr wd)| and |lr clip u| (one rounded product and one fma),
against the oracle's fp64 update of the same partitions.
"""

from __future__ import annotations

import numpy as np
import pytest

import muon_newton_schulz_step_amd as M
import oracle.muon_oracle as O
import workloads as W
from gpu_util import SENTINEL, host, sentinel_partitions, to_device, workspace

pytestmark = pytest.mark.gpu

SHAPES = [(300, 200), (130, 520), (257, 257), (96, 640), (1, 33), (40, 1), (512, 700)]


@pytest.fixture(scope="module")
def torch():
    t = pytest.importorskip("torch")
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    M.load()
    return t


def _group(shapes, R=3, precision="bf16", grad_dtype="fp32", cap=0):
    offsets, P = O.pack_layout(shapes, R, 16)
    g = M.MuonGroup(shapes, offsets=offsets, num_partitions=R, partition_numel=P, method="standard",
                    precision=precision, grad_dtype=grad_dtype, max_inflight_bytes=cap)
    return g, offsets, P


def _grads(torch, shapes, seed, dtype="fp32", scale=1.0):
    out = []
    for i, s in enumerate(shapes):
        a = W.gaussian(s, seed + 10 * i, 0.02) * np.float32(scale)
        out.append(to_device(W.f32_to_bf16_bits(a) if dtype == "bf16" else a, dtype))
    return out


def _flag(torch, v):
    return torch.tensor([v], dtype=torch.int32, device="cuda:0")


def test_grad_scale_cancels_loss_scale_bitwise(torch):
    g, offsets, P = _group(SHAPES)
    ws_t, ws = workspace(g.workspace_bytes)
    runs = []
    for S in (1.0, 2.0 ** 14):
        moms = [torch.zeros(s, dtype=torch.float32, device="cuda:0") for s in SHAPES]
        parts = sentinel_partitions(3, P)
        for step in range(2):
            gr = _grads(torch, SHAPES, 100 * step, scale=S)
            g.step(gr, moms, parts, ws, grad_scale=1.0 / S)
        torch.cuda.synchronize()
        runs.append(([host(p) for p in parts], [host(m) for m in moms]))
    for a, b in zip(runs[0][0] + runs[0][1], runs[1][0] + runs[1][1]):
        np.testing.assert_array_equal(a, b)


def test_skip_flag_leaves_momentum_and_partitions(torch):
    g, offsets, P = _group(SHAPES)
    ws_t, ws = workspace(g.workspace_bytes)
    moms = [torch.zeros(s, dtype=torch.float32, device="cuda:0") for s in SHAPES]
    parts = sentinel_partitions(3, P)
    g.step(_grads(torch, SHAPES, 1), moms, parts, ws)
    torch.cuda.synchronize()
    mom0, part0 = [host(m).copy() for m in moms], [host(p).copy() for p in parts]
    # a discarded step with non-finite gradients: nothing changes
    bad = _grads(torch, SHAPES, 2)
    bad[0][0, 0] = float("inf")
    flag = _flag(torch, 0)
    g.check_finite(bad, "fp32", flag, ws)
    torch.cuda.synchronize()
    assert int(flag.item()) == 1
    g.step(bad, moms, parts, ws, skip_flag=flag)
    torch.cuda.synchronize()
    for a, b in zip([host(m) for m in moms] + [host(p) for p in parts], mom0 + part0):
        np.testing.assert_array_equal(a, b)
    # flag 0: the same as a plain step from the same state
    good = _grads(torch, SHAPES, 3)
    flag.zero_()
    moms_b = [m.clone() for m in moms]
    parts_b = [p.clone() for p in parts]
    g.step(good, moms, parts, ws, skip_flag=flag)
    g.step(good, moms_b, parts_b, ws)
    torch.cuda.synchronize()
    for a, b in zip(moms + parts, moms_b + parts_b):
        np.testing.assert_array_equal(host(a), host(b))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_check_finite(torch, dtype):
    g, offsets, P = _group(SHAPES, grad_dtype=dtype)
    ws_t, ws = workspace(g.workspace_bytes)
    flag = _flag(torch, 7)
    clean = _grads(torch, SHAPES, 5, dtype)
    g.check_finite(clean, dtype, flag, ws)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    rng = np.random.default_rng(9)
    for bad_value in (float("inf"), float("-inf"), float("nan")):
        for i in (0, 4, 6):
            gr = _grads(torch, SHAPES, 5, dtype)
            r, c = SHAPES[i]
            gr[i][int(rng.integers(r)), int(rng.integers(c))] = bad_value
            g.check_finite(gr, dtype, flag, ws)
            torch.cuda.synchronize()
            assert int(flag.item()) == 1, (bad_value, i)
            g.check_finite(clean, dtype, flag, ws)
            torch.cuda.synchronize()
            assert int(flag.item()) == 0


def _params(torch, P, R, seed):
    out = []
    for r in range(R):
        a = W.gaussian((P,), seed + r, 0.5)
        out.append(to_device(a, "fp32"))
    return out


@np.errstate(invalid="ignore")
def _check_params(got, want, before, parts, lr, wd, clip):
    decay = 1.0 - lr * wd
    for r in range(len(got)):
        scale = np.maximum(np.abs(before[r].astype(np.float64) * decay),
                           np.abs(lr * clip * parts[r].astype(np.float64)))
        bound = 2.0 * np.spacing(scale.astype(np.float32)).astype(np.float64)
        diff = np.abs(got[r].astype(np.float64) - want[r].astype(np.float64))
        ok = (diff <= bound) | (got[r].view(np.uint32) == want[r].view(np.uint32))
        assert np.all(ok), f"partition {r}: worst {np.max(diff / np.maximum(bound, 1e-45)):.2f} x bound"


@pytest.mark.parametrize("max_norm", [0.0, 1e6, 0.05])
def test_apply_update_vs_oracle(torch, max_norm):
    g, offsets, P = _group(SHAPES)
    ws_t, ws = workspace(g.workspace_bytes)
    moms = [torch.zeros(s, dtype=torch.float32, device="cuda:0") for s in SHAPES]
    parts = [torch.zeros(P, dtype=torch.float32, device="cuda:0") for _ in range(3)]
    g.step(_grads(torch, SHAPES, 11), moms, parts, ws)
    params = _params(torch, P, 3, 40)
    # padding of the params carries a sentinel that must survive
    sent = np.array([SENTINEL], dtype=np.uint32).view(np.float32)[0]
    covered = np.zeros(3 * P, dtype=bool)
    for (r, c), off in zip(SHAPES, offsets):
        covered[off:off + r * c] = True
    flat = torch.cat(params).cpu().numpy()
    flat[~covered] = sent
    params = [to_device(flat[r * P:(r + 1) * P], "fp32") for r in range(3)]
    before = [host(p).copy() for p in params]
    nc = torch.zeros(2, dtype=torch.float32, device="cuda:0")
    lr, wd = 0.02, 0.1
    g.apply_update(params, parts, lr, wd, max_norm, ws, norm_clip_out=nc)
    torch.cuda.synchronize()
    hp = [host(p) for p in parts]
    want, norm, clip = O.apply_update(before, hp, SHAPES, offsets, lr, wd, max_norm)
    got_norm, got_clip = (float(v) for v in nc.cpu().numpy())
    assert got_norm == pytest.approx(norm, rel=1e-6)
    assert got_clip == pytest.approx(clip, rel=1e-6)
    if max_norm == 0.05:
        assert clip < 1.0
    got = [host(p) for p in params]
    _check_params(got, want, before, hp, lr, wd, clip)
    gflat = np.concatenate(got).view(np.uint32)
    assert np.all(gflat[~covered] == SENTINEL), "padding of the parameters was written"


def test_apply_update_skip_and_determinism(torch):
    g, offsets, P = _group(SHAPES)
    ws_t, ws = workspace(g.workspace_bytes)
    moms = [torch.zeros(s, dtype=torch.float32, device="cuda:0") for s in SHAPES]
    parts = [torch.zeros(P, dtype=torch.float32, device="cuda:0") for _ in range(3)]
    g.step(_grads(torch, SHAPES, 12), moms, parts, ws)
    params = _params(torch, P, 3, 50)
    before = [host(p).copy() for p in params]
    nc1 = torch.zeros(2, dtype=torch.float32, device="cuda:0")
    nc2 = torch.zeros(2, dtype=torch.float32, device="cuda:0")
    g.apply_update(params, parts, 0.1, 0.1, 0.5, ws, skip_flag=_flag(torch, 1), norm_clip_out=nc1)
    torch.cuda.synchronize()
    for a, b in zip([host(p) for p in params], before):
        np.testing.assert_array_equal(a, b)
    assert float(nc1.abs().sum()) == 0.0
    g.apply_update(params, parts, 0.1, 0.1, 0.5, ws, norm_clip_out=nc1)
    g.apply_update(params, parts, 0.1, 0.1, 0.5, ws, norm_clip_out=nc2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(nc1), host(nc2))


def test_checkpoint_continuation_bitwise(torch):
    """Interrupted vs uninterrupted: three steps (each followed by the
    parameter update) against one step, a checkpoint of momenta and
    parameters to the host, a new plan and workspace, the restore, and two
    more steps.  Everything bit for bit."""
    shapes, R = SHAPES[:4], 2
    grads = [_grads(torch, shapes, 1000 * k) for k in range(3)]

    def fresh():
        g, offsets, P = _group(shapes, R)
        ws_t, ws = workspace(g.workspace_bytes)
        return g, P, ws_t, ws

    def run(g, ws, P, moms, params, ks):
        parts = [torch.zeros(P, dtype=torch.float32, device="cuda:0") for _ in range(R)]
        for k in ks:
            g.step(grads[k], moms, parts, ws)
            g.apply_update(params, parts, 0.05, 0.01, 1.0, ws)
        torch.cuda.synchronize()
        return parts

    g, P, ws_t, ws = fresh()
    moms_a = [torch.zeros(s, dtype=torch.float32, device="cuda:0") for s in shapes]
    params_a = _params(torch, P, R, 60)
    parts_a = run(g, ws, P, moms_a, params_a, [0, 1, 2])

    g1, P1, ws_t1, ws1 = fresh()
    moms_b = [torch.zeros(s, dtype=torch.float32, device="cuda:0") for s in shapes]
    params_b = _params(torch, P1, R, 60)
    run(g1, ws1, P1, moms_b, params_b, [0])
    ckpt = ([host(m).copy() for m in moms_b], [host(p).copy() for p in params_b])
    g1.close()
    del ws_t1, moms_b, params_b
    g2, P2, ws_t2, ws2 = fresh()
    moms_c = [to_device(m, "fp32") for m in ckpt[0]]
    params_c = [to_device(p, "fp32") for p in ckpt[1]]
    parts_c = run(g2, ws2, P2, moms_c, params_c, [1, 2])
    for a, b in zip(moms_a + params_a + parts_a, moms_c + params_c + parts_c):
        np.testing.assert_array_equal(host(a), host(b))


def test_apply_update_after_multi_wave_step(torch):
    """A step cut into one workspace wave per matrix leaves the same update
    partials, so the norm, the clip factor and the parameters agree with the
    one-wave run (the partial sums are grouped differently: fp64 rounding
    only)."""
    outs = []
    for cap in (0, 1):
        g, offsets, P = _group(SHAPES, cap=cap)
        if cap:
            assert g.stats()["waves"] == len(SHAPES)
        ws_t, ws = workspace(g.workspace_bytes)
        moms = [torch.zeros(s, dtype=torch.float32, device="cuda:0") for s in SHAPES]
        parts = [torch.zeros(P, dtype=torch.float32, device="cuda:0") for _ in range(3)]
        g.step(_grads(torch, SHAPES, 77), moms, parts, ws)
        params = _params(torch, P, 3, 80)
        nc = torch.zeros(2, dtype=torch.float32, device="cuda:0")
        g.apply_update(params, parts, 0.03, 0.05, 0.2, ws, norm_clip_out=nc)
        torch.cuda.synchronize()
        outs.append(([host(p) for p in parts], [host(p) for p in params], host(nc)))
    for a, b in zip(outs[0][0], outs[1][0]):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_allclose(outs[1][2], outs[0][2], rtol=1e-6)
    for a, b in zip(outs[0][1], outs[1][1]):
        np.testing.assert_allclose(b, a, rtol=1e-6, atol=1e-9)


@pytest.mark.parametrize("precision", ["fp32", "bf16"])
def test_training_trajectory_vs_oracle(torch, precision):
    """Three optimizer steps run as a mixed-precision training loop runs them,
    against the oracle's muon_step / apply_update sequence on the same bits.
    Gradients are made under loss scale S = 2^12 and handed in with
    grad_scale 1/S; before every step the overflow check writes the device
    skip flag that the step and the parameter update both read; the middle
    step's gradients hold an Inf, so that step is discarded on both sides;
    every step ends with the clipped parameter update.

    Checked after every step: the flag against the oracle's own finiteness
    decision; momenta within 3 fp32 spacings of |beta m| + |(1-beta) g|;
    every matrix and 256 x 256 block of the update within the Newton-Schulz
    tolerance; the norm within that tolerance; the parameters against the
    oracle's update of the GPU's own inputs (2 fp32 spacings).  At the end the
    parameters against the all-oracle trajectory, within the bound the
    update tolerance implies: sum over kept steps of lr clip ||u|| (2 tol)
    (a relative error tol in u and at most tol in the clip factor), plus 2
    fp32 spacings of |p| per step."""
    from gpu_util import assert_tiles_within
    tol = {"fp32": 1e-4, "bf16": 2e-2}[precision]
    shapes, R = SHAPES, 3
    g, offsets, P = _group(shapes, R, precision=precision, grad_dtype="fp32")
    ws_t, ws = workspace(g.workspace_bytes)
    S = 2.0 ** 12
    lr, wd, max_norm = 0.02, 0.1, 0.5
    beta = float(np.float32(0.95))
    host_grads = []
    for k in range(3):
        gk = [W.gaussian(s, 5000 + 100 * k + i, 0.02) * np.float32(S) for i, s in enumerate(shapes)]
        if k == 1:
            gk[2][7, 11] = np.float32(np.inf)
        host_grads.append(gk)
    p0 = [W.gaussian((P,), 6000 + r, 0.5) for r in range(R)]

    # HIP path
    moms = [torch.zeros(s, dtype=torch.float32, device="cuda:0") for s in shapes]
    parts = [torch.zeros(P, dtype=torch.float32, device="cuda:0") for _ in range(R)]
    params = [to_device(p, "fp32") for p in p0]
    flag = _flag(torch, 0)
    nc = torch.zeros(2, dtype=torch.float32, device="cuda:0")

    # oracle
    opt = O.MuonOptions(beta=beta, method="standard", eps=float(np.float32(O.NORM_EPS)))
    state = O.init_state(shapes)
    parts_o = [np.zeros(P, dtype=np.float32) for _ in range(R)]
    params_o = [p.copy() for p in p0]
    bound_u = 0.0
    for k in range(3):
        dev = [to_device(x, "fp32") for x in host_grads[k]]
        g.check_finite(dev, "fp32", flag, ws)
        before = [host(p).copy() for p in params]
        g.step(dev, moms, parts, ws, skip_flag=flag, grad_scale=1.0 / S)
        g.apply_update(params, parts, lr, wd, max_norm, ws, skip_flag=flag, norm_clip_out=nc)
        torch.cuda.synchronize()

        skip = not all(np.all(np.isfinite(x)) for x in host_grads[k])
        assert int(flag.item()) == int(skip), f"step {k}: overflow flag"
        grads64 = [O.as_f64(x, "fp32") for x in host_grads[k]]
        scale_terms = None if skip else [np.abs(beta * m.astype(np.float64)) + np.abs((1 - beta) * gg / S)
                                         for m, gg in zip(state.momenta, grads64)]
        O.muon_step(grads64, state, shapes, [0] * len(shapes), offsets, R, P, opt, partitions=parts_o,
                    grad_scale=1.0 / S, skip=skip)
        params_o, norm_o, clip_o = O.apply_update(params_o, parts_o, shapes, offsets, lr, wd, max_norm, skip=skip)

        for i, (got, want) in enumerate(zip([host(m) for m in moms], state.momenta)):
            if skip:
                continue
            bound = 3 * np.spacing(scale_terms[i].astype(np.float32)).astype(np.float64)
            diff = np.abs(got.astype(np.float64) - want.astype(np.float64))
            assert np.all(diff <= bound), f"step {k} momentum {i}"
        hp = [host(p) for p in parts]
        for i, (r, c) in enumerate(shapes):
            got_u = O.gather_from_partitions(hp, offsets[i], r, c)
            want_u = O.gather_from_partitions(parts_o, offsets[i], r, c)
            err = O.rel_frobenius(got_u, want_u)
            assert err <= tol, f"step {k} matrix {i}: update rel err {err:.3e}"
            assert_tiles_within(got_u, want_u, tol, f"step {k} matrix {i}")
        got_p = [host(p) for p in params]
        if skip:
            for a, b in zip(got_p, before):
                np.testing.assert_array_equal(a, b)
            continue
        got_norm, got_clip = (float(v) for v in host(nc))
        assert got_norm == pytest.approx(norm_o, rel=tol)
        assert got_clip == pytest.approx(clip_o, rel=2 * tol)
        assert clip_o < 1.0, "max_norm is meant to clip"
        want_p, _, clip_g = O.apply_update(before, hp, shapes, offsets, lr, wd, max_norm)
        _check_params(got_p, want_p, before, hp, lr, wd, clip_g)
        bound_u += lr * clip_o * norm_o * 2 * tol

    st = g.stats()
    n = len(shapes)
    assert st["steps"] == 3 and st["ns_invocations"] == 3 * n and st["flagged_steps"] == 3
    assert state.steps == 2 and state.ns_invocations == 2 * n
    got_p = np.concatenate([host(p) for p in params]).astype(np.float64)
    want_p = np.concatenate(params_o).astype(np.float64)
    spacing = np.linalg.norm(2 * np.spacing(np.abs(want_p).astype(np.float32)).astype(np.float64)) * 2
    dev_p = float(np.linalg.norm(got_p - want_p))
    print(f"{precision}: parameter deviation {dev_p:.3e} against bound {bound_u + spacing:.3e}")
    assert dev_p <= bound_u + spacing
