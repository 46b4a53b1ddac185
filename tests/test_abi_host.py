"""The C-ABI library on the host: it loads, exports every declared symbol,
validates plans, lays out owned runs like a brute-force enumeration, and
rejects bad calls before touching the device (no GPU needed)."""

from __future__ import annotations

import os
import re

import numpy as np
import pytest

import muon_newton_schulz_step_amd as M
from muon_newton_schulz_step_amd import _lib
from oracle_pins import brute_force_index_map, runs_to_index_map

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "muon.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = M.load()
    declared = _declared_symbols()
    assert set(declared) == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    for code, name in _lib.STATUS.items():
        assert M.muon_status_string(code) == name


def test_default_options():
    o = M.muon_default_options()
    assert o.beta == pytest.approx(0.95) and o.nesterov == 1 and o.ns_steps == 5
    assert (o.a, o.b, o.c) == pytest.approx((3.4445, -4.7750, 2.0315))
    assert o.method == 0 and o.precision == 1
    assert o.max_inflight_bytes == 24 << 30 and o.schedule == 0 and o.reserved == 0


def _group(shapes, **kw):
    return M.MuonGroup(shapes, **kw)


@pytest.mark.parametrize("bad,code", [
    (dict(shapes=[(0, 4)]), "MUON_ERR_INVALID_ARG"),
    (dict(shapes=[(4, 4)], heads=[3]), "MUON_ERR_UNSUPPORTED"),
    (dict(shapes=[(4, 4)], heads=[-1]), "MUON_ERR_INVALID_ARG"),
    (dict(shapes=[(4, 4)], ns_steps=-1), "MUON_ERR_INVALID_ARG"),
    (dict(shapes=[(4, 4)], beta=1.0), "MUON_ERR_INVALID_ARG"),
    (dict(shapes=[(4, 4)], beta=-0.1), "MUON_ERR_INVALID_ARG"),
    (dict(shapes=[(4, 4), (2, 2)], offsets=[0, 15], partition_numel=32), "MUON_ERR_LAYOUT"),
    (dict(shapes=[(4, 4)], offsets=[20], partition_numel=32), "MUON_ERR_LAYOUT"),
    (dict(shapes=[(4, 4)], offsets=[-1], partition_numel=32), "MUON_ERR_LAYOUT"),
])
def test_plan_rejects(bad, code):
    with pytest.raises(M.MuonError) as ei:
        _group(**bad)
    assert ei.value.name == code
    assert M.muon_last_error()


def test_plan_rejects_unknown_enums():
    o = M.muon_default_options()
    lay = M.muon_layout(16, 1, 0)
    for field, val in (("method", 2), ("precision", 5), ("grad_dtype", 7), ("nesterov", 2)):
        o2 = M.muon_default_options()
        setattr(o2, field, val)
        with pytest.raises(M.MuonError) as ei:
            M.muon_plan_create([(4, 4, 0, 0)], o2, lay)
        assert ei.value.name == "MUON_ERR_INVALID_ARG"
    with pytest.raises(M.MuonError):
        M.muon_plan_create([], o, lay)


@pytest.mark.parametrize("seed", range(6))
def test_runs_match_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 6))
    shapes = [(int(rng.integers(1, 20)), int(rng.integers(1, 20))) for _ in range(n)]
    R = int(rng.integers(1, 5))
    offsets, P = M.pack_layout(shapes, R, 16, interior_align=bool(seed % 2))
    g = _group(shapes, offsets=offsets, num_partitions=R, partition_numel=P)
    for i, (r, c) in enumerate(shapes):
        runs = [(p, off, first, length) for p, off, first, length in g.runs(i)]
        assert runs_to_index_map(runs, r * c) == brute_force_index_map(offsets[i], r * c, P)


def test_tiny_layout_runs():
    shapes = [(17, 13), (9, 17)]
    offsets, P = M.pack_layout(shapes, 2, 16)
    assert offsets == [0, 221] and P == 192
    g = _group(shapes, num_partitions=2)
    assert g.runs(0) == [(0, 0, 0, 192), (1, 0, 192, 29)]
    assert g.runs(1) == [(1, 29, 0, 153)]


def test_problems_orientation_and_heads():
    g = _group([(17, 13), (9, 17), (4096, 1024), (256, 64)], heads=[0, 0, 0, 2])
    probs = g.problems()
    assert [(q["matrix"], q["head"], q["m"], q["n"], q["transposed"]) for q in probs] == [
        (0, 0, 13, 17, True), (1, 0, 9, 17, False), (2, 0, 1024, 4096, True),
        (3, 0, 64, 128, True), (3, 1, 64, 128, True)]
    m, n = 1024, 4096
    assert probs[2]["flops"] == pytest.approx(5 * (4 * m * m * n + 2 * m ** 3))
    gg = _group([(1024, 4096)], method="gram")
    assert gg.problems()[0]["flops"] == pytest.approx(4 * m * m * n + 17 * 2 * m ** 3)


def test_workspace_waves_bound_memory():
    shapes = [(512, 512)] * 8
    g1 = _group(shapes)
    assert g1.stats()["waves"] == 1
    cap = g1.workspace_bytes // 3
    g2 = _group(shapes, max_inflight_bytes=cap)
    assert g2.stats()["waves"] > 1
    assert g2.workspace_bytes < g1.workspace_bytes
    assert {q["wave"] for q in g2.problems()} == set(range(g2.stats()["waves"]))


def test_step_validation_fails_before_device():
    g = _group([(8, 8), (4, 12)], grad_dtype="fp32", precision="fp32")
    ws_bytes = g.workspace_bytes
    base = 1 << 40
    ws = base + (1 << 30)
    grads = [base, base + 4096]
    moms = [base + 8192, base + 12288]
    parts = [base + 16384]
    # NULL entries
    with pytest.raises(M.MuonError) as ei:
        M.muon_step(g.plan, [0, grads[1]], moms, parts, ws, ws_bytes, 0)
    assert ei.value.name == "MUON_ERR_INVALID_ARG"
    # overlapping buffers
    with pytest.raises(M.MuonError) as ei:
        M.muon_step(g.plan, grads, [grads[0] + 16, moms[1]], parts, ws, ws_bytes, 0)
    assert ei.value.name == "MUON_ERR_ALIAS"
    # partition overlapping the workspace
    with pytest.raises(M.MuonError) as ei:
        M.muon_step(g.plan, grads, moms, [ws + 256], ws, ws_bytes, 0)
    assert ei.value.name == "MUON_ERR_ALIAS"
    # workspace too small / unaligned / missing
    for w, wb in ((ws, ws_bytes - 1), (ws + 8, ws_bytes), (0, ws_bytes)):
        with pytest.raises(M.MuonError) as ei:
            M.muon_step(g.plan, grads, moms, parts, w, wb, 0)
        assert ei.value.name == "MUON_ERR_WORKSPACE"
    # accumulate and scatter validate the same way
    with pytest.raises(M.MuonError) as ei:
        M.muon_accumulate(g.plan, [moms[0], moms[0]], grads, "fp32", True, ws, ws_bytes, 0)
    assert ei.value.name == "MUON_ERR_ALIAS"
    with pytest.raises(M.MuonError) as ei:
        M.muon_scatter(g.plan, grads, 7, parts, ws, ws_bytes, 0)
    assert ei.value.name == "MUON_ERR_INVALID_ARG"
    assert g.stats()["steps"] == 0 and g.stats()["ns_invocations"] == 0


def test_step_ex_check_and_apply_validation_fails_before_device():
    g = _group([(8, 8), (4, 12)], grad_dtype="fp32", precision="fp32")
    ws_bytes = g.workspace_bytes
    base = 1 << 40
    ws = base + (1 << 30)
    grads = [base, base + 4096]
    moms = [base + 8192, base + 12288]
    parts = [base + 16384]
    params = [base + 32768]
    flag = base + 65536
    # grad_scale must be finite
    for bad in (float("inf"), float("nan")):
        with pytest.raises(M.MuonError) as ei:
            M.muon_step_ex(g.plan, grads, moms, parts, flag, bad, ws, ws_bytes, 0)
        assert ei.value.name == "MUON_ERR_INVALID_ARG"
    # the skip flag may not overlap another buffer of the call
    with pytest.raises(M.MuonError) as ei:
        M.muon_step_ex(g.plan, grads, moms, parts, moms[0] + 4, 1.0, ws, ws_bytes, 0)
    assert ei.value.name == "MUON_ERR_ALIAS"
    # finite check: unknown dtype, NULL flag, flag inside a gradient
    with pytest.raises(M.MuonError) as ei:
        M.muon_check_finite(g.plan, grads, 5, flag, ws, ws_bytes, 0)
    assert ei.value.name == "MUON_ERR_INVALID_ARG"
    with pytest.raises(M.MuonError) as ei:
        M.muon_check_finite(g.plan, grads, "fp32", 0, ws, ws_bytes, 0)
    assert ei.value.name == "MUON_ERR_INVALID_ARG"
    with pytest.raises(M.MuonError) as ei:
        M.muon_check_finite(g.plan, grads, "fp32", grads[0] + 8, ws, ws_bytes, 0)
    assert ei.value.name == "MUON_ERR_ALIAS"
    # apply: no step has run on this workspace yet
    with pytest.raises(M.MuonError) as ei:
        M.muon_apply_update(g.plan, params, parts, 0.1, 0.0, 1.0, None, None, ws, ws_bytes, 0)
    assert ei.value.name == "MUON_ERR_INVALID_ARG"
    assert "no muon_step" in str(ei.value)
    # non-finite hyper-parameters, NULL entries
    with pytest.raises(M.MuonError) as ei:
        M.muon_apply_update(g.plan, params, parts, float("nan"), 0.0, 1.0, None, None, ws, ws_bytes, 0)
    assert ei.value.name == "MUON_ERR_INVALID_ARG"
    with pytest.raises(M.MuonError) as ei:
        M.muon_apply_update(g.plan, [0], parts, 0.1, 0.0, 1.0, None, None, ws, ws_bytes, 0)
    assert ei.value.name == "MUON_ERR_INVALID_ARG"


def test_plan_rejects_tile_index_overflow():
    # GEMM tile coordinates are int16 on the device: a side needing more than
    # 32767 tiles of 128 is refused at plan creation, one tile short is not
    with pytest.raises(M.MuonError) as ei:
        _group([(1 << 23, 1)], precision="fp32", grad_dtype="fp32")
    assert ei.value.name == "MUON_ERR_UNSUPPORTED"
    assert "32767" in M.muon_last_error()
    g = _group([(32767 * 128, 1)], precision="fp32", grad_dtype="fp32")
    assert g.problems()[0]["n"] == 32767 * 128
    g.close()


def test_binding_refuses_short_pointer_tables():
    g = _group([(8, 8), (4, 12)], grad_dtype="fp32", precision="fp32", num_partitions=2)
    base = 1 << 40
    ws = base + (1 << 30)
    grads, moms, parts = [base, base + 4096], [base + 8192, base + 12288], [base + 16384, base + 20480]
    with pytest.raises(ValueError, match="grads"):
        M.muon_step(g.plan, grads[:1], moms, parts, ws, g.workspace_bytes, 0)
    with pytest.raises(ValueError, match="partitions"):
        M.muon_step_ex(g.plan, grads, moms, parts[:1], None, 1.0, ws, g.workspace_bytes, 0)
    with pytest.raises(ValueError, match="grad_mb"):
        M.muon_accumulate(g.plan, moms, grads + [base], "fp32", True, ws, g.workspace_bytes, 0)
    with pytest.raises(ValueError, match="params"):
        M.muon_apply_update(g.plan, [base], parts, 0.1, 0.0, 1.0, None, None, ws, g.workspace_bytes, 0)
    assert g.stats()["steps"] == 0 and g.stats()["flagged_steps"] == 0


def test_group_checks_tensor_arguments():
    torch = pytest.importorskip("torch")
    shapes = [(8, 8), (4, 12)]
    g = _group(shapes, grad_dtype="bf16", precision="bf16")
    grads = [torch.zeros(s, dtype=torch.bfloat16) for s in shapes]
    moms = [torch.zeros(s, dtype=torch.float32) for s in shapes]
    parts = [torch.zeros(g.partition_numel, dtype=torch.float32)]
    ws = torch.zeros(g.workspace_bytes, dtype=torch.uint8)
    # wrong gradient dtype (fp32 handed to a bf16 plan)
    with pytest.raises(ValueError, match="dtype"):
        g.step([m.clone() for m in moms], moms, parts, ws)
    # a transposed view
    bad = [grads[0].t(), grads[1]]
    with pytest.raises(ValueError, match="contiguous"):
        g.step(bad, moms, parts, ws)
    # wrong element count, wrong buffer count
    with pytest.raises(ValueError, match="elements"):
        g.step(grads, [moms[0], torch.zeros(4, 11)], parts, ws)
    with pytest.raises(ValueError, match="buffers"):
        g.step(grads[:1], moms[:1], parts, ws)
    with pytest.raises(ValueError, match="partitions"):
        g.step(grads, moms, [torch.zeros(g.partition_numel - 1)], ws)
    # well-formed host tensors are still refused before any device call
    with pytest.raises(ValueError, match="host tensor"):
        g.step(grads, moms, parts, ws)
    # a workspace tensor smaller than the byte count claimed for it
    small = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="workspace"):
        M.muon_step(g.plan, [1 << 40, (1 << 40) + 4096], [(1 << 40) + 8192, (1 << 40) + 12288],
                    [(1 << 40) + 16384], small, g.workspace_bytes, 0)
    assert g.stats()["steps"] == 0


def test_noalloc_scratch_size_matches_header_and_refuses_large_plans():
    text = open(os.path.join(ROOT, "include", "muon.h")).read()
    m = re.search(r"#define MUON_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES
    g = _group([(4096, 4096)])
    assert g.workspace_bytes > _lib.NOALLOC_SCRATCH_BYTES
    base = 1 << 40
    with pytest.raises(M.MuonError) as ei:
        M.muon_step_noalloc(g.plan, [base], [base + (1 << 26)], [base + (1 << 28)], None, 1.0, 0)
    assert ei.value.name == "MUON_ERR_WORKSPACE"
    assert "max_inflight_bytes" in M.muon_last_error()
    assert g.stats()["steps"] == 0
