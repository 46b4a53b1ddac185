"""The large-tile GEMM ties its accumulators in place with inline-asm MFMAs,
whose result latency the compiler does not see.  Compile the kernel to gfx950
assembly (CPU only, no device) and check that nothing reads an accumulator
written by one of those MFMAs before the result can have landed: every
non-MFMA read, and every MFMA reading it as an A or B operand, must follow
the write by at least MIN_WAIT wait states on every path, branches included.  The
checker itself is pinned on small listings with a planted early read."""

from __future__ import annotations

import importlib.util
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "muon_newton_schulz_step_amd", "csrc")

# An 8-pass XDL result needs about 11 wait states before a VALU or memory
# instruction may read it; 18 leaves margin.  An intervening MFMA counts 4
# (the fewest cycles between two MFMA issues).
MIN_WAIT = 18
MFMA_WAIT = 4
# A VALU write of a VGPR or AGPR needs 2 wait states before an MFMA reads it;
# the compiler inserts them for its own MFMAs only.  Checked with margin.
VALU_WAIT = 3

_STORES = ("ds_write", "global_store", "buffer_store", "scratch_store", "flat_store")


def _regs(tok: str) -> set[str]:
    """Registers a VGPR or AGPR operand names, as 'v12' / 'a12'."""
    tok = tok.strip()
    m = re.match(r"([av])\[(\d+):(\d+)\]$", tok)
    if m:
        return {m.group(1) + str(i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([av])(\d+)$", tok)
    return {tok} if m else set()


def _agprs(tok: str) -> set[int]:
    tok = tok.strip()
    m = re.match(r"a\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"a(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def early_reads(listing: str) -> list[str]:
    """Two hazards the compiler cannot see through inline asm, along every
    path: a read of an AGPR written by an inline-asm MFMA fewer than MIN_WAIT
    wait states earlier, and an inline-asm MFMA reading (as A, B or C) a
    register that a VALU instruction (v_accvgpr_write / mov included) wrote
    fewer than VALU_WAIT wait states earlier.  The state is carried through
    fall-through and into every branch target (the largest wait still owed
    wins where paths meet), and each function is swept until the states at
    its labels settle, so loop back-edges are covered too."""
    funcs: list[list[str]] = []
    for raw in listing.splitlines():
        s = raw.strip()
        if re.match(r"^_Z\w+:", s):
            funcs.append([])
            continue
        if funcs:
            funcs[-1].append(s)
    bad: set[str] = set()
    for body in funcs:
        # owed: ("m", agpr) -> wait states an asm MFMA result still needs;
        #       ("w", reg)  -> wait states a VALU write still needs before an asm MFMA reads it
        at_label: dict[str, dict[tuple, int]] = {}
        for _ in range(8):
            changed = False
            owed: dict[tuple, int] | None = {}  # None = unreachable
            in_asm = False

            def spend(n_mfma: int, n_valu: int) -> None:
                for key in list(owed):
                    owed[key] -= n_mfma if key[0] == "m" else n_valu
                    if owed[key] <= 0:
                        del owed[key]

            def send(target: str) -> None:
                nonlocal changed
                cur = at_label.setdefault(target, {})
                for key, w in owed.items():
                    if cur.get(key, 0) < w:
                        cur[key] = w
                        changed = True

            for s in body:
                if s.startswith(";;#ASMSTART"):
                    in_asm = True
                    continue
                if s.startswith(";;#ASMEND"):
                    in_asm = False
                    continue
                m = re.match(r"^(\.LBB\w+):", s)
                if m:
                    merged = dict(at_label.get(m.group(1), {}))
                    for key, w in (owed or {}).items():
                        merged[key] = max(merged.get(key, 0), w)
                    owed = merged
                    continue
                if not s or s.startswith(";") or s.startswith(".") or owed is None:
                    continue
                op = s.split()[0]
                args = [a for a in re.split(r"[ ,]+", s[len(op):].strip()) if a]
                if op.startswith("s_branch") or op.startswith("s_cbranch"):
                    send(args[0])
                    if op.startswith("s_branch"):
                        owed = None
                    continue
                if op in ("s_endpgm", "s_setpc_b64"):
                    owed = None
                    continue
                if op.startswith("v_mfma"):
                    for a in args[1:3]:
                        if any(("m", r) in owed for r in _agprs(a)):
                            bad.add(s)
                    if in_asm and any(("w", r) in owed for a in args[1:4] for r in _regs(a)):
                        bad.add(s)
                    spend(MFMA_WAIT, 1)
                    for r in (_agprs(args[0]) if args else set()):
                        if in_asm:
                            owed[("m", r)] = MIN_WAIT
                        else:
                            owed.pop(("m", r), None)
                    continue
                n = int(args[0], 0) + 1 if op == "s_nop" else 1
                spend(n, n)
                reads = args if op.startswith(_STORES) else args[1:]
                for a in reads:
                    if any(("m", r) in owed for r in _agprs(a)):
                        bad.add(s)
                if args and not op.startswith(_STORES) and not op.startswith("s_"):
                    for r in _agprs(args[0]):
                        owed.pop(("m", r), None)
                    if op.startswith("v_"):
                        for r in _regs(args[0]):
                            owed[("w", r)] = VALU_WAIT
            if not changed:
                break
    return sorted(bad)


def test_checker_catches_a_planted_early_read():
    ok = "\n".join([
        "_Zk:",
        ";;#ASMSTART", "v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]", ";;#ASMEND",
        "s_nop 15", "s_nop 7",
        "v_accvgpr_read_b32 v8, a0",
    ])
    early = "\n".join([
        "_Zk:",
        ";;#ASMSTART", "v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]", ";;#ASMEND",
        "v_accvgpr_mov_b32 a9, a2",
    ])
    builtin = "\n".join([
        "_Zk:",
        "v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]",
        "v_accvgpr_read_b32 v8, a0",
    ])
    branch_only = "\n".join([
        "_Zk:",
        ";;#ASMSTART", "v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]", ";;#ASMEND",
        "s_branch .LBB0_2",
        ".LBB0_1:",
        "v_accvgpr_read_b32 v8, a0",
    ])
    via_branch = "\n".join([
        "_Zk:",
        ";;#ASMSTART", "v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]", ";;#ASMEND",
        "s_cbranch_scc1 .LBB0_2",
        "s_nop 15", "s_nop 7",
        "s_endpgm",
        ".LBB0_2:",
        "v_accvgpr_read_b32 v8, a1",
    ])
    back_edge = "\n".join([
        "_Zk:",
        ".LBB0_1:",
        "v_accvgpr_read_b32 v8, a2",
        "s_nop 15", "s_nop 7",
        ";;#ASMSTART", "v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]", ";;#ASMEND",
        "s_cbranch_scc1 .LBB0_1",
        "s_endpgm",
    ])
    valu_then_asm = "\n".join([
        "_Zk:",
        "v_accvgpr_write_b32 a3, v9",
        ";;#ASMSTART", "v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]", ";;#ASMEND",
    ])
    valu_spaced = "\n".join([
        "_Zk:",
        "v_mov_b32 v5, v9",
        "s_nop 2",
        ";;#ASMSTART", "v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]", ";;#ASMEND",
    ])
    valu_then_builtin = "\n".join([
        "_Zk:",
        "v_accvgpr_write_b32 a3, v9",
        "v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]",
    ])
    assert early_reads(valu_then_asm) == ["v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]"]
    assert early_reads(valu_spaced) == []
    assert early_reads(valu_then_builtin) == []   # the compiler covers its own MFMAs
    assert early_reads(ok) == []
    assert early_reads(early) == ["v_accvgpr_mov_b32 a9, a2"]
    assert early_reads(builtin) == []       # the compiler covers its own MFMAs
    assert early_reads(branch_only) == []   # the read is on no path from the MFMA
    assert early_reads(via_branch) == ["v_accvgpr_read_b32 v8, a1"]
    assert early_reads(back_edge) == ["v_accvgpr_read_b32 v8, a2"]


def test_large_tile_gemm_reads_no_asm_mfma_result_early(tmp_path):
    hipcc = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)
    if hipcc is None:
        pytest.skip("hipcc is not available")
    out = str(tmp_path / "k_gemm256.s")
    # the library's own compile flags, so the listing is the code it ships
    spec = importlib.util.spec_from_file_location("_muon_build", os.path.join(ROOT, "muon_newton_schulz_step_amd", "build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    cmd = [hipcc, *build.COMMON, "--cuda-device-only", "-S", os.path.join(CSRC, "k_gemm256.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    listing = open(out).read()
    n_asm_mfma = len(re.findall(r";;#ASMSTART\s*\n\s*v_mfma", listing))
    assert n_asm_mfma > 0, "the kernel no longer uses inline-asm MFMAs; this check is moot"
    bad = early_reads(listing)
    assert bad == [], f"{len(bad)} early reads, e.g. {bad[:5]}"
