"""The large-tile GEMM ties its accumulators in place with inline-asm MFMAs,
whose result latency the compiler does not see.  Compile the kernel to gfx950
assembly (CPU only, no device) and check that nothing reads an accumulator
written by one of those MFMAs before the result can have landed: every
non-MFMA read, and every MFMA reading it as an A or B operand, must follow
the write by at least MIN_WAIT wait states along the fall-through code.  The
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
    states earlier, scanning each function's code in layout order and
    dropping the state at labels that only a branch reaches."""
    bad: list[str] = []
    pending: dict[int, int] = {}  # agpr -> wait-state clock at the asm MFMA write
    clock = 0
    in_asm = False
    prev = ""
    for raw in listing.splitlines():
        s = raw.strip()
        if re.match(r"^_Z\w+:", s):
            pending, clock, prev = {}, 0, ""
            continue
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if re.match(r"^\.LBB\w+:", s):
            if prev in ("s_branch", "s_endpgm", "s_setpc_b64"):
                pending = {}
            continue
        if not s or s.startswith(";") or s.startswith("."):
            continue
        op = s.split()[0]
        prev = op
        args = [a for a in re.split(r"[ ,]+", s[len(op):].strip()) if a]
        if op.startswith("v_mfma"):
            for a in args[1:3]:
                for r in _agprs(a):
                    if r in pending and clock - pending[r] < MIN_WAIT:
                        bad.append(s)
            clock += MFMA_WAIT
            dst = _agprs(args[0]) if args else set()
            for r in dst:
                if in_asm:
                    pending[r] = clock
                else:
                    pending.pop(r, None)
            continue
        if op == "s_nop":
            clock += int(args[0], 0) + 1
            continue
        clock += 1
        reads = args if op.startswith(_STORES) else args[1:]
        for a in reads:
            for r in _agprs(a):
                if r in pending and clock - pending[r] < MIN_WAIT:
                    bad.append(s)
        if args and not op.startswith(_STORES) and not op.startswith("s_"):
            for r in _agprs(args[0]):
                pending.pop(r, None)
    return bad


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
    assert early_reads(ok) == []
    assert early_reads(early) == ["v_accvgpr_mov_b32 a9, a2"]
    assert early_reads(builtin) == []       # the compiler covers its own MFMAs
    assert early_reads(branch_only) == []   # not reached by fall-through


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
