"""Full-size groups in the launch configuration the benchmark times, checked
against the oracle on sampled matrices (the oracle computes them one by one
in fp64), plus properties that hold for every matrix of the group.

Inputs are drawn on the GPU from a seeded torch generator, matrix by matrix;
the sampled matrices' inputs are copied to the host for the oracle, so both
sides see the same bits.
"""

from __future__ import annotations

import time

import numpy as np
import pytest

import muon_newton_schulz_step_amd as M
import oracle.muon_oracle as O
import workloads as W
from gpu_util import assert_tiles_within

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

TOL_BF16 = 2e-2


@pytest.fixture(scope="module")
def torch():
    t = pytest.importorskip("torch")
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    M.load()
    return t


def _views(flat, shapes):
    out, off = [], 0
    for (r, c) in shapes:
        out.append(flat[off:off + r * c].view(r, c))
        off += r * c
    return out


def _fill(torch, views, shapes, seed, sigma, dtype):
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(seed)
    for v, (r, c) in zip(views, shapes):
        v.copy_(torch.randn((r, c), generator=gen, device="cuda:0", dtype=torch.float32).mul_(sigma).to(dtype))


def _host_f64(torch, t):
    return t.to(torch.float64).cpu().numpy()


def _run_group(torch, wl, method, sample, gas_buffers=1):
    """Run one step of the full group; return (sampled updates from the
    partitions, sampled oracle updates, flat partitions tensor, plan)."""
    offsets, P = M.pack_layout(wl.shapes, wl.num_partitions, wl.align)
    step_dtype = "fp32" if wl.gas > 1 else wl.micro_dtype
    g = M.MuonGroup(wl.shapes, heads=wl.heads, offsets=offsets, num_partitions=wl.num_partitions,
                    partition_numel=P, method=method, precision="bf16", grad_dtype=step_dtype)
    total = wl.numel
    mdt = torch.bfloat16 if wl.micro_dtype == "bf16" else torch.float32
    mb_flat = torch.empty(total, dtype=mdt, device="cuda:0")
    mb = _views(mb_flat, wl.shapes)
    mom_flat = torch.zeros(total, dtype=torch.float32, device="cuda:0")
    mom = _views(mom_flat, wl.shapes)
    parts_flat = torch.zeros(wl.num_partitions * P, dtype=torch.float32, device="cuda:0")
    parts = [parts_flat[r * P:(r + 1) * P] for r in range(wl.num_partitions)]
    ws = torch.empty(g.workspace_bytes, dtype=torch.uint8, device="cuda:0")
    assert ws.data_ptr() % 256 == 0
    host_mb = {i: [] for i in sample}
    if wl.gas > 1:
        acc_flat = torch.empty(total, dtype=torch.float32, device="cuda:0")
        acc = _views(acc_flat, wl.shapes)
        for k in range(wl.gas):
            _fill(torch, mb, wl.shapes, 1000 * wl.config_id + 17 * k, wl.sigma, mdt)
            for i in sample:
                host_mb[i].append(_host_f64(torch, mb[i]))
            g.accumulate(acc, mb, wl.micro_dtype, k == 0, ws)
            torch.cuda.synchronize()
        grads = acc
    else:
        _fill(torch, mb, wl.shapes, 1000 * wl.config_id, wl.sigma, mdt)
        for i in sample:
            host_mb[i].append(_host_f64(torch, mb[i]))
        grads = mb
    g.step(grads, mom, parts, ws)
    torch.cuda.synchronize()
    got, want = {}, {}
    opt = O.MuonOptions(method=method, beta=float(np.float32(0.95)), eps=float(np.float32(O.NORM_EPS)))
    for i in sample:
        r, c = wl.shapes[i]
        t0 = time.perf_counter()
        got[i] = parts_flat[offsets[i]:offsets[i] + r * c].view(r, c).cpu().numpy()
        state = O.init_state([(r, c)])
        res = O.muon_step([O.accumulate(host_mb[i])], state, [(r, c)], [wl.heads[i]], [0], 1, r * c, opt)
        want[i] = res.updates[0]
        del host_mb[i]
        print(f"  oracle {wl.name} {method} matrix {i} {r}x{c}: {time.perf_counter() - t0:.1f} s", flush=True)
    return got, want, parts_flat, offsets, P, g


def _check_sampled(wl, method, got, want, sample, tile=256):
    """Matrix-level and tile x tile block-level relative Frobenius error of
    every sampled matrix within the bf16 tolerance (tile 128 for head-split
    groups: one block per head and 128 columns)."""
    worst = 0.0
    for i in sample:
        err = O.rel_frobenius(got[i], want[i])
        label = f"{wl.name} ({method}), matrix {i} {wl.shapes[i]}"
        blk = assert_tiles_within(got[i], want[i], TOL_BF16, label, tile=tile)
        print(f"{label}: rel err {err:.3e}, worst {tile}x{tile} block {blk:.3e}", flush=True)
        assert err <= TOL_BF16, label
        worst = max(worst, err)
    return worst


def _finite_and_covered(torch, parts_flat, wl, offsets):
    assert bool(torch.isfinite(parts_flat[:sum(r * c for r, c in wl.shapes)]).all())
    # every matrix received a non-trivial update of the expected size: the
    # unscaled output has Frobenius norm sqrt(sum f^5(sigma)^2) <= 1.21 sqrt(m)
    for i, ((r, c), off) in enumerate(zip(wl.shapes, offsets)):
        u = parts_flat[off:off + r * c].double()
        h = wl.heads[i] or 1
        m = min(r // h, c)
        scale = O.shape_scale(r, c)
        nrm = float(u.norm()) / scale
        assert 0.3 * (h * m) ** 0.5 < nrm < 1.21 * (h * m) ** 0.5, (i, nrm)


def test_h1024_full_group_all_matrices(torch):
    wl = W.h1024()
    sample = list(range(len(wl.shapes)))
    got, want, parts_flat, offsets, P, g = _run_group(torch, wl, "standard", sample)
    worst = _check_sampled(wl, "standard", got, want, sample)
    print(f"h1024 12-layer group, all 72 matrices: worst rel err {worst:.3e}")
    assert g.stats()["ns_invocations"] == len(wl.shapes)
    # single partition, tail padding after the last matrix is untouched (zeros here)
    assert float(parts_flat[sum(r * c for r, c in wl.shapes):].abs().sum()) == 0.0


@pytest.mark.parametrize("method", ["gram", "standard"])
def test_per_head_full_group_sampled(torch, method):
    """The per-head group in the bench's launch configuration: the 2048 head
    blocks on the fused kernel beside the o-matrices on the large-tile one."""
    wl = W.per_head()
    sample = [0, 2, len(wl.shapes) - 2]   # layer 0 q (32 heads), layer 0 o (unsplit), layer 31 k (32 heads)
    got, want, parts_flat, offsets, P, g = _run_group(torch, wl, method, sample)
    _check_sampled(wl, method, got, want, sample, tile=128)
    _finite_and_covered(torch, parts_flat, wl, offsets)


@pytest.mark.timeout(900)
def test_llama7b_full_group_sampled(torch):
    """The Llama-7B group (224 matrices, gas 4 into fp32, 8 partitions) in the
    standard form: layer 0 and layer 31 in full (q, k, v, o 4096x4096, gate,
    up 4096x11008, down 11008x4096 transposed with shape scale 1.64), about
    90 s of fp64 oracle, plus the size-independent checks on every matrix."""
    wl = W.llama7b()
    L = len(wl.shapes)
    sample = list(range(7)) + list(range(L - 7, L))
    got, want, parts_flat, offsets, P, g = _run_group(torch, wl, "standard", sample)
    _check_sampled(wl, "standard", got, want, sample)
    _finite_and_covered(torch, parts_flat, wl, offsets)
    st = g.stats()
    assert st["ns_invocations"] == 224 and st["accumulations"] == 4 and st["steps"] == 1


@pytest.mark.timeout(900)
def test_share70b_full_group_sampled(torch):
    """The 70B single-GPU share (8 layers, 56 matrices, 6.85 G elements) in
    the bench's launch configuration.  The oracle checks the first layer's q
    (8192 x 8192, about 30 s of fp64 oracle) and gate (8192 x 28672: the
    longest K loop of the large-tile kernel, about 90 s), and the k and v
    projections (8192 x 1024, tall: 1024 x 8192 blocks on the large-tile
    kernel, shape scale 2.83) of the first and last layer; every matrix of
    the group gets the size-independent checks."""
    wl = W.share70b()
    L = len(wl.shapes)
    sample = [0, 1, 2, 4, L - 5]          # layer 0 q, k, v, gate; layer 7 k
    got, want, parts_flat, offsets, P, g = _run_group(torch, wl, "standard", sample)
    _check_sampled(wl, "standard", got, want, sample)
    _finite_and_covered(torch, parts_flat, wl, offsets)
    assert g.stats()["ns_invocations"] == L


def test_llama7b_full_group_gram_sampled(torch):
    """The Llama-7B group in the Gram form: its 4096-row blocks run the
    split-bf16 m x m chain on the large-tile kernel.  Same sample as the
    standard form (every matrix kind)."""
    torch.cuda.empty_cache()
    wl = W.llama7b()
    sample = [0, 4, len(wl.shapes) - 1]
    got, want, parts_flat, offsets, P, g = _run_group(torch, wl, "gram", sample)
    _check_sampled(wl, "gram", got, want, sample)
    _finite_and_covered(torch, parts_flat, wl, offsets)
    assert g.stats()["ns_invocations"] == 224


@pytest.mark.timeout(900)
def test_share70b_full_group_gram_sampled(torch):
    """The 70B share in the Gram form: the first layer's q (8192 x 8192, the
    split-bf16 chain at its largest; about 40 s of fp64 oracle), the k / v
    projections of the first and last layer (1024 x 8192 blocks, chain of
    1024 x 1024 products) and the last layer's down projection (28672 x 8192:
    tall, transposed, shape scale 1.87; about 60 s), plus the
    size-independent checks on every matrix."""
    torch.cuda.empty_cache()
    wl = W.share70b()
    L = len(wl.shapes)
    sample = [0, 1, 2, L - 5, L - 1]
    got, want, parts_flat, offsets, P, g = _run_group(torch, wl, "gram", sample)
    _check_sampled(wl, "gram", got, want, sample)
    _finite_and_covered(torch, parts_flat, wl, offsets)
    assert g.stats()["ns_invocations"] == L
