"""muon_step_noalloc (the library's static device workspace) against
muon_step_ex (a caller workspace), through the C ABI on cuda:0.

The two entry points launch the same kernels on the same inputs, so their
momenta and partitions must agree bit for bit.  Calls come in a row on one
process: a group, then a smaller group (the array keeps the first call's
contents), then the first group again in the Gram form, then a discarded
step (device skip flag) and a loss-scaled one.  Last, the step captured once
into a graph and replayed on new gradients, with eager steps between the
replays: every replay equals an eager step on the same inputs.
"""

from __future__ import annotations

import numpy as np
import pytest

import muon_newton_schulz_step_amd as M
import oracle.muon_oracle as O
import workloads as W
from gpu_util import host, sentinel_partitions, to_device, workspace

pytestmark = pytest.mark.gpu

BIG = [(300, 200), (130, 520), (257, 257), (96, 640), (1, 33), (40, 1), (512, 700)]
SMALL = [(64, 96), (17, 13), (200, 33)]


@pytest.fixture(scope="module")
def torch():
    t = pytest.importorskip("torch")
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    M.load()
    return t


def _both(torch, shapes, method, seed, R=3, grad_scale=1.0, skip=None, mom_seed=None, cap=0):
    """One step through each entry point from the same state; returns the
    two (partitions, momenta) results as host arrays."""
    offsets, P = O.pack_layout(shapes, R, 16)
    g = M.MuonGroup(shapes, offsets=offsets, num_partitions=R, partition_numel=P, method=method,
                    precision="bf16", grad_dtype="bf16", max_inflight_bytes=cap)
    assert g.workspace_bytes <= M._lib.NOALLOC_SCRATCH_BYTES
    grads_h = [W.make_grad(s, seed + 10 * i, 0.02, "bf16") for i, s in enumerate(shapes)]
    mom_h = [W.warm_momentum(s, (mom_seed or seed) + i, 0.02) for i, s in enumerate(shapes)]
    flag = None if skip is None else torch.tensor([int(skip)], dtype=torch.int32, device="cuda:0")
    out = []
    for noalloc in (False, True):
        grads = [to_device(x, "bf16") for x in grads_h]
        moms = [to_device(m, "fp32") for m in mom_h]
        parts = sentinel_partitions(R, P)
        if noalloc:
            g.step_noalloc(grads, moms, parts, skip_flag=flag, grad_scale=grad_scale)
        else:
            ws_t, ws = workspace(g.workspace_bytes)
            g.step(grads, moms, parts, ws, skip_flag=flag, grad_scale=grad_scale)
        torch.cuda.synchronize()
        out.append(([host(p) for p in parts], [host(m) for m in moms]))
    st = g.stats()
    assert st["steps"] == 2 and st["ns_invocations"] == 2 * len(shapes)
    g.close()
    return out, mom_h


def _equal(a, b, label):
    for k, (x, y) in enumerate(zip(a[0] + a[1], b[0] + b[1])):
        np.testing.assert_array_equal(x.view(np.uint32), y.view(np.uint32), err_msg=f"{label}: buffer {k}")


def test_noalloc_matches_workspace_entry_point(torch):
    (ref, got), _ = _both(torch, BIG, "standard", 100)
    _equal(ref, got, "group of 7, standard")
    # the second call, on a smaller group, reuses the array the first left
    (ref, got), _ = _both(torch, SMALL, "standard", 200)
    _equal(ref, got, "group of 3, standard")
    (ref, got), _ = _both(torch, BIG, "gram", 300)
    _equal(ref, got, "group of 7, gram")
    # eight 1024 x 1024 matrices need more than the array; capped, they run
    # in waves that fit
    (ref, got), _ = _both(torch, [(1024, 1024)] * 8, "standard", 600, R=2, cap=30 << 20)
    _equal(ref, got, "eight 1024^2 in waves")


def test_noalloc_skip_flag_and_grad_scale(torch):
    (ref, got), mom_h = _both(torch, SMALL, "standard", 400, skip=1)
    _equal(ref, got, "discarded step")
    for m, m0 in zip(got[1], mom_h):
        np.testing.assert_array_equal(m, m0)
    (ref, got), _ = _both(torch, SMALL, "standard", 500, grad_scale=2.0 ** -10)
    _equal(ref, got, "scaled step")


def test_noalloc_refuses_a_plan_beyond_the_array(torch):
    g = M.MuonGroup([(4096, 4096)], precision="bf16", grad_dtype="bf16")
    assert g.workspace_bytes > M._lib.NOALLOC_SCRATCH_BYTES
    grads = [torch.zeros((4096, 4096), dtype=torch.bfloat16, device="cuda:0")]
    moms = [torch.zeros((4096, 4096), dtype=torch.float32, device="cuda:0")]
    parts = [torch.zeros(g.partition_numel, dtype=torch.float32, device="cuda:0")]
    with pytest.raises(M.MuonError) as ei:
        g.step_noalloc(grads, moms, parts)
    assert ei.value.name == "MUON_ERR_WORKSPACE"
    assert g.stats()["steps"] == 0
    g.close()


def test_noalloc_step_replays_from_a_graph(torch):
    # A graph is what a caller that cannot allocate records: the step's
    # launches (tables included, as kernel arguments) are captured once and
    # replayed; each replay re-uploads the captured tables into the array.
    shapes = [(300, 200), (128, 640), (512, 700), (17, 13)]
    offsets, P = O.pack_layout(shapes, 2, 16)
    g = M.MuonGroup(shapes, offsets=offsets, num_partitions=2, partition_numel=P, method="standard",
                    precision="bf16", grad_dtype="bf16")
    assert g.workspace_bytes <= M._lib.NOALLOC_SCRATCH_BYTES
    grads = [torch.empty(s, dtype=torch.bfloat16, device="cuda:0") for s in shapes]
    moms = [to_device(W.warm_momentum(s, 800 + i, 0.02), "fp32").reshape(s) for i, s in enumerate(shapes)]
    parts = sentinel_partitions(2, P)

    def load_grads(k):
        for i, s in enumerate(shapes):
            grads[i].copy_(to_device(W.make_grad(s, 900 + 10 * k + i, 0.02, "bf16"), "bf16").reshape(s))

    # eager warm-up on a side stream, then capture on the graph's stream
    load_grads(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g.step_noalloc(grads, moms, parts)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.step_noalloc(grads, moms, parts)
    torch.cuda.synchronize()
    for k in range(1, 4):
        load_grads(k)
        torch.cuda.synchronize()
        # the eager step on copies of the same state and inputs
        ref_grads = [x.clone() for x in grads]
        ref_moms = [m.clone() for m in moms]
        ref_parts = [p.clone() for p in parts]
        g.step_noalloc(ref_grads, ref_moms, ref_parts)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _equal(([host(p) for p in ref_parts], [host(m) for m in ref_moms]),
               ([host(p) for p in parts], [host(m) for m in moms]), f"replay {k}")
    graph.reset()
    g.close()
