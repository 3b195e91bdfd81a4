"""The launch tables the library builds on the host from its copy of the
routing (the split shrink's XCD placement, the feature-tile tables of the
one-kernel delta and of the split-K expand half), checked on the CPU: a
program that compiles the library source with tests/host_tables_check.cpp
calls the builders on fixed and random routings and checks that every unit
of work appears exactly once.  A duplicated unit would not change any result
on the GPU (it recomputes the same values), so the parity tests cannot see
it."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_tables_cover_every_unit_once(tmp_path):
    csrc = os.path.join(ROOT, "segmented_rank_gemv_amd", "csrc")
    exe = tmp_path / "host_tables_check"
    cmd = [HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O0", "-I", os.path.join(ROOT, "include"), "-I", csrc,
           os.path.join(ROOT, "tests", "host_tables_check.cpp"), os.path.join(csrc, "lora_host.cpp"),
           os.path.join(csrc, "lora_cache.cpp"), "-o", str(exe)]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr[-3000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("bad 0"), r.stdout[-3000:]
