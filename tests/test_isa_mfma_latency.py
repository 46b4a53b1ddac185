"""The large-tile GEMM ties its accumulators in place with inline-asm MFMAs,
whose result latency the compiler does not see.  Compile the kernel to gfx950
assembly (CPU only, no device) and check that nothing reads an accumulator
written by one of those MFMAs before the result can have landed: every
non-MFMA read, and every MFMA reading it as an A or B operand, must follow
the write by at least MIN_WAIT wait states on every path, branches included.  The
checker itself is pinned on small listings with a planted early read."""

from __future__ import annotations

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

_STORES = ("ds_write", "global_store", "buffer_store", "scratch_store", "flat_store")


def _agprs(tok: str) -> set[int]:
    tok = tok.strip()
    m = re.match(r"a\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"a(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def early_reads(listing: str) -> list[str]:
    """Reads of AGPRs written by an inline-asm MFMA fewer than MIN_WAIT wait
    states earlier, along every path: the state is carried through
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
        at_label: dict[str, dict[int, int]] = {}
        for _ in range(8):
            changed = False
            owed: dict[int, int] | None = {}  # agpr -> wait states still owed; None = unreachable
            in_asm = False

            def spend(n: int) -> None:
                for r in list(owed):
                    owed[r] -= n
                    if owed[r] <= 0:
                        del owed[r]

            def send(target: str) -> None:
                nonlocal changed
                cur = at_label.setdefault(target, {})
                for r, w in owed.items():
                    if cur.get(r, 0) < w:
                        cur[r] = w
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
                    for r, w in (owed or {}).items():
                        merged[r] = max(merged.get(r, 0), w)
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
                        if any(r in owed for r in _agprs(a)):
                            bad.add(s)
                    spend(MFMA_WAIT)
                    for r in (_agprs(args[0]) if args else set()):
                        if in_asm:
                            owed[r] = MIN_WAIT
                        else:
                            owed.pop(r, None)
                    continue
                spend(int(args[0], 0) + 1 if op == "s_nop" else 1)
                reads = args if op.startswith(_STORES) else args[1:]
                for a in reads:
                    if any(r in owed for r in _agprs(a)):
                        bad.add(s)
                if args and not op.startswith(_STORES) and not op.startswith("s_"):
                    for r in _agprs(args[0]):
                        owed.pop(r, None)
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
    cmd = [hipcc, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           os.path.join(CSRC, "k_gemm256.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    listing = open(out).read()
    n_asm_mfma = len(re.findall(r";;#ASMSTART\s*\n\s*v_mfma", listing))
    assert n_asm_mfma > 0, "the kernel no longer uses inline-asm MFMAs; this check is moot"
    bad = early_reads(listing)
    assert bad == [], f"{len(bad)} early reads, e.g. {bad[:5]}"
