"""The fused Newton-Schulz of small blocks (bf16 operands, small side
64..128: one workgroup runs a block's whole iteration), in both forms,
against the oracle: head blocks of 128 rows at the per-head shape and ragged ones, tall
blocks (output stored transposed), several 128-column chunks with a ragged
last chunk, a single chunk, every step count, and the same blocks beside a
large-tile matrix (the second stream).  Per matrix and per 128 x 128 block
(one head block's rows), relative Frobenius error within the bf16 bound."""

from __future__ import annotations

import numpy as np
import pytest

import muon_newton_schulz_step_amd as M
import oracle.muon_oracle as O
import workloads as W
from gpu_util import SENTINEL, assert_tiles_within, run_steps

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.load()
    yield


def _run(shapes, heads, method, steps_ns=5, R=2, cid=91, label=""):
    offsets, P = O.pack_layout(shapes, R, 16)
    g = M.MuonGroup(shapes, heads=heads, offsets=offsets, num_partitions=R, partition_numel=P, method=method,
                    precision="bf16", grad_dtype="bf16", ns_steps=steps_ns)
    micro = [[[W.make_grad(s, W.grad_seed(cid, i, 0, t), 0.02, "bf16") for i, s in enumerate(shapes)]]
             for t in range(2)]
    m0 = [W.warm_momentum(s, 300 + i, 0.02) for i, s in enumerate(shapes)]
    parts, moms = run_steps(g, micro, "bf16", momenta0=m0, use_accumulate=False)

    state = O.init_state(shapes)
    state.momenta = [m.astype(np.float32).copy() for m in m0]
    opt = O.MuonOptions(beta=float(np.float32(0.95)), nesterov=True, method=method, steps=steps_ns,
                        eps=float(np.float32(O.NORM_EPS)))
    sentinel = np.array([SENTINEL], dtype=np.uint32).view(np.float32)[0]
    oparts = [np.full(P, sentinel, dtype=np.float32) for _ in range(R)]
    res = None
    for step in micro:
        grads = [O.as_f64(step[0][i], "bf16") for i in range(len(shapes))]
        res = O.muon_step(grads, state, shapes, heads, offsets, R, P, opt, partitions=oparts)
    worst = 0.0
    for i, (r, c) in enumerate(shapes):
        got = O.gather_from_partitions(parts, offsets[i], r, c)
        err = O.rel_frobenius(got, res.updates[i])
        worst = max(worst, err)
        assert err <= TOL, f"{label} matrix {i} {r}x{c}: rel err {err:.3e} > {TOL}"
        assert_tiles_within(got, res.updates[i], TOL, f"{label} matrix {i} {r}x{c}", tile=128)
    # padding untouched
    flat = np.concatenate(parts).view(np.uint32)
    covered = np.zeros(flat.size, dtype=bool)
    for (r, c), off in zip(shapes, offsets):
        covered[off:off + r * c] = True
    assert np.all(flat[~covered] == SENTINEL), "padding was written"
    print(f"{label}: worst rel err {worst:.3e}")
    return g


@pytest.mark.parametrize("method", ["gram", "standard"])
def test_head_blocks_and_small_sides(method):
    shapes = [
        (512, 4096),   # 4 head blocks of 128 x 4096 (the per-head block shape), 32 chunks
        (384, 1000),   # 3 head blocks of 128 x 1000: ragged last chunk
        (100, 1000),   # m = 100
        (64, 129),     # m = 64, one column past a chunk
        (65, 65),      # square, one chunk
        (127, 300),
        (700, 128),    # tall: output stored transposed
        (1000, 96),    # tall, m = 96, ragged
        (256, 77),     # 2 tall head blocks of 128 x 77
    ]
    heads = [4, 3, 0, 0, 0, 0, 0, 0, 2]
    g = _run(shapes, heads, method, label=f"fused blocks/{method}")
    probs = g.problems()
    assert all(64 <= q["m"] <= 128 for q in probs) and any(q["transposed"] for q in probs)


@pytest.mark.parametrize("steps_ns", [1, 2, 3])
@pytest.mark.parametrize("method", ["gram", "standard"])
def test_head_step_counts(method, steps_ns):
    _run([(128, 640), (200, 128), (96, 96)], [0, 0, 0], method, steps_ns=steps_ns, cid=93,
         label=f"T={steps_ns}/{method}")


@pytest.mark.parametrize("method", ["gram", "standard"])
def test_head_blocks_beside_large_tiles(method):
    # the head blocks run on the second stream while the 512 x 768 matrix
    # takes the large-tile kernel
    _run([(512, 768), (1024, 2048), (768, 512)], [0, 8, 0], method, cid=95, label=f"beside large tiles/{method}")
