"""The C ABI from plain C: include/muon.h compiles as C99 and as C++17 with
every warning an error, and a C99 client linked against the built library
plans a group on the host, reads it back and frees it (no GPU needed)."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

import muon_newton_schulz_step_amd as M
from muon_newton_schulz_step_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")
SRC = os.path.join(ROOT, "tests", "host", "c_client.c")


def _tool(name):
    path = shutil.which(name)
    if not path:
        pytest.skip(f"{name} not found")
    return path


def test_header_compiles_as_c99_and_cxx17(tmp_path):
    for cmd in ([_tool("gcc"), "-std=c99", "-x", "c"], [_tool("g++"), "-std=c++17", "-x", "c++"]):
        r = subprocess.run(cmd + ["-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", "-I", INC, SRC],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_c_client_links_and_plans_on_the_host(tmp_path):
    M.load()  # the library is built
    libdir = os.path.dirname(_lib.LIB_PATH)
    exe = str(tmp_path / "c_client")
    r = subprocess.run([_tool("gcc"), "-std=c99", "-Wall", "-Werror", "-I", INC, SRC, "-o", exe, "-L", libdir,
                        "-l:" + os.path.basename(_lib.LIB_PATH), f"-Wl,-rpath,{libdir}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stderr
    assert "c client ok" in run.stdout
