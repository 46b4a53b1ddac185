"""The persistent schedule of the large-tile blocks (one launch per wave
runs every product of every bf16 block with m >= 256, workgroups taking
tiles from a queue of their XCD and waiting on a per-block counter for the
block's previous product) against one launch per product.

Each tile's arithmetic is the same in both schedules, so the momenta and
partitions must agree bit for bit: in both forms, with the Gram form's
lean class (m >= 2048), head blocks of 256 rows, tall and ragged blocks,
the 128-tile and fused small blocks beside them on the second stream, and
under a workspace cap that cuts the group into waves (one persistent launch
per wave and group).  One group is also checked against the oracle, the
allocation-free entry point against the workspace one, and a discarded
step (device skip flag) against the untouched state."""

from __future__ import annotations

import numpy as np
import pytest

import muon_newton_schulz_step_amd as M
import oracle.muon_oracle as O
import workloads as W
from gpu_util import SENTINEL, assert_tiles_within, host, run_steps, sentinel_partitions, to_device, workspace

pytestmark = pytest.mark.gpu

MIXED = [
    (512, 768),     # large tiles, one tile row past a multiple
    (1024, 2048),   # 4 head blocks of 256 x 2048 (large tiles)
    (768, 3000),    # ragged last column tile
    (2048, 1024),   # tall: the block is 1024 x 2048, output stored transposed
    (300, 4096),    # m = 300: a ragged 44-row edge tile row
    (2048, 2304),   # m = 2048: the Gram form's lean class
    (512, 4096),    # 4 head blocks of 128 rows: the fused kernel, second stream
    (200, 300),     # the 128-tile kernel, second stream
    (1000, 96),     # tall, fused
]
MIXED_HEADS = [0, 4, 0, 0, 0, 0, 4, 0, 0]


@pytest.fixture(scope="module")
def torch():
    t = pytest.importorskip("torch")
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    M.load()
    return t


def _group(shapes, heads, method, schedule, R=2, cap=0):
    offsets, P = O.pack_layout(shapes, R, 16)
    return M.MuonGroup(shapes, heads=heads, offsets=offsets, num_partitions=R, partition_numel=P, method=method,
                       precision="bf16", grad_dtype="bf16", ns_steps=5, max_inflight_bytes=cap, schedule=schedule)


def _micro(shapes, cid, steps=2):
    return [[[W.make_grad(s, W.grad_seed(cid, i, 0, t), 0.02, "bf16") for i, s in enumerate(shapes)]]
            for t in range(steps)]


def _moms(shapes):
    return [W.warm_momentum(s, 500 + i, 0.02) for i, s in enumerate(shapes)]


def _both(shapes, heads, method, cid, cap=0):
    out = {}
    for sched in ("launches", "persistent"):
        g = _group(shapes, heads, method, sched, cap=cap)
        out[sched] = (g,) + run_steps(g, _micro(shapes, cid), "bf16", momenta0=_moms(shapes), use_accumulate=False)
    return out


def _same(out, label):
    (_, pa, ma), (_, pb, mb) = out["launches"], out["persistent"]
    for i, (a, b) in enumerate(zip(pa, pb)):
        d = int(np.count_nonzero(a.view(np.uint32) != b.view(np.uint32)))
        assert d == 0, f"{label}: partition {i}: {d} words differ between the schedules"
    for i, (a, b) in enumerate(zip(ma, mb)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{label}: momentum {i} differs"


@pytest.mark.parametrize("method", ["standard", "gram"])
def test_persistent_equals_launches(torch, method):
    out = _both(MIXED, MIXED_HEADS, method, cid=61)
    g = out["persistent"][0]
    assert g.stats()["waves"] == 1
    _same(out, f"mixed group/{method}")


@pytest.mark.parametrize("method", ["standard", "gram"])
def test_persistent_waves(torch, method):
    # a cap of a third of the uncapped workspace: several waves, each with
    # its own queues and counters
    shapes = [(512, 768), (768, 1024), (1024, 1024), (300, 2000), (256, 256), (640, 512)]
    heads = [0] * len(shapes)
    cap = _group(shapes, heads, method, "persistent").workspace_bytes // 3
    out = _both(shapes, heads, method, cid=63, cap=cap)
    assert out["persistent"][0].stats()["waves"] >= 2
    _same(out, f"waves/{method}")


@pytest.mark.parametrize("method", ["standard", "gram"])
def test_persistent_against_oracle(torch, method):
    shapes = [(300, 520), (256, 257), (700, 512), (96, 300)]
    heads = [0] * len(shapes)
    R = 2
    offsets, P = O.pack_layout(shapes, R, 16)
    g = _group(shapes, heads, method, "persistent", R=R)
    micro = _micro(shapes, cid=65)
    m0 = _moms(shapes)
    parts, _ = run_steps(g, micro, "bf16", momenta0=m0, use_accumulate=False)
    state = O.init_state(shapes)
    state.momenta = [m.astype(np.float32).copy() for m in m0]
    opt = O.MuonOptions(beta=float(np.float32(0.95)), nesterov=True, method=method, steps=5,
                        eps=float(np.float32(O.NORM_EPS)))
    sentinel = np.array([SENTINEL], dtype=np.uint32).view(np.float32)[0]
    oparts = [np.full(P, sentinel, dtype=np.float32) for _ in range(R)]
    res = None
    for step in micro:
        grads = [O.as_f64(step[0][i], "bf16") for i in range(len(shapes))]
        res = O.muon_step(grads, state, shapes, heads, offsets, R, P, opt, partitions=oparts)
    for i, (r, c) in enumerate(shapes):
        got = O.gather_from_partitions(parts, offsets[i], r, c)
        err = O.rel_frobenius(got, res.updates[i])
        assert err <= 2e-2, f"matrix {i} {r}x{c}: rel err {err:.3e}"
        assert_tiles_within(got, res.updates[i], 2e-2, f"persistent/{method} matrix {i}")


def test_persistent_noalloc_and_skip(torch):
    shapes = [(512, 700), (300, 300), (130, 520)]
    R = 2
    offsets, P = O.pack_layout(shapes, R, 16)
    g = M.MuonGroup(shapes, offsets=offsets, num_partitions=R, partition_numel=P, method="standard",
                    precision="bf16", grad_dtype="bf16", schedule="persistent")
    grads_h = [W.make_grad(s, 71 + i, 0.02, "bf16") for i, s in enumerate(shapes)]
    mom_h = [W.warm_momentum(s, 81 + i, 0.02) for i, s in enumerate(shapes)]
    out = []
    for noalloc in (False, True):
        grads = [to_device(x, "bf16") for x in grads_h]
        moms = [to_device(m, "fp32") for m in mom_h]
        parts = sentinel_partitions(R, P)
        if noalloc:
            g.step_noalloc(grads, moms, parts)
        else:
            ws_t, ws = workspace(g.workspace_bytes)
            g.step(grads, moms, parts, ws)
        torch.cuda.synchronize()
        out.append(([host(p) for p in parts], [host(m) for m in moms]))
    for a, b in zip(out[0][0] + out[0][1], out[1][0] + out[1][1]):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "allocation-free step differs"
    # a discarded step: the persistent launch does nothing, state untouched
    flag = torch.tensor([1], dtype=torch.int32, device="cuda:0")
    grads = [to_device(x, "bf16") for x in grads_h]
    moms = [to_device(m, "fp32") for m in mom_h]
    parts = sentinel_partitions(R, P)
    ws_t, ws = workspace(g.workspace_bytes)
    g.step(grads, moms, parts, ws, skip_flag=flag)
    torch.cuda.synchronize()
    for p in parts:
        assert np.all(host(p).view(np.uint32) == SENTINEL), "a discarded step wrote the partitions"
    for m, m0 in zip(moms, mom_h):
        assert np.array_equal(host(m), m0.astype(np.float32)), "a discarded step moved the momentum"
