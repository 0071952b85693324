"""Schedule tables of phase 1 checked on the host (no GPU).

The planner (attention_fia_fwd_amd/csrc/fia_plan.cpp) is compiled with
stand-ins for its device hooks together with tests/plan_tables_check.cpp,
which captures the table image phase 1 would upload and checks that every
prefill row block is scheduled exactly once, that the zero-fill items cover
exactly the padding rows, that each XCD bucket is in longest-first order, that
every block-sparse (batch, head, row slice) is one workgroup inside one q block,
and that the decode pieces of every segment (GQA decode, MLA decode with and
without the sliding band) tile its kv range exactly within the per-wave quota
(the invariants the GPU parity tests rely on)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_schedule_tables_of_phase1(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "plan_tables_check")
    cmd = [cxx, "-O1", "-std=c++17", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "attention_fia_fwd_amd", "csrc"),
           os.path.join(ROOT, "tests", "plan_tables_check.cpp"),
           os.path.join(ROOT, "attention_fia_fwd_amd", "csrc", "fia_plan.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0 and run.stdout.strip().endswith("all ok"), run.stdout[-4000:]
