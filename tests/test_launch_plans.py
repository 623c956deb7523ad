"""Launch plans of the product kernels, checked on the CPU.

tests/plan_check.cpp includes ternary_quantized_linear_amd/csrc/bl_plan.h (the host-side
planning the launchers use), replays each kernel's index arithmetic over thousands of
shapes -- grouped decode layers, ragged N and K, every supported K range, 1 and 2 token
blocks, split-K token counts, BitDelta row counts -- on several device sizes, and checks
that every row, 16-byte chunk, row block, K segment, k-tile and tile is covered exactly
once, that LDS stays within a CU and that 32-bit buffer offsets stay in range.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_launch_plans_cover_every_shape(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "plan_check")
    r = subprocess.run([gxx, "-std=c++17", "-O2", "-Wall", "-o", exe,
                        os.path.join(HERE, "plan_check.cpp")], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().startswith("ok"), r.stdout[-4000:] + r.stderr
