"""Phase 1 under random, mostly invalid, inputs (host only, no GPU).

tests/phase1_fuzz.cpp is compiled together with the planner
(attention_fia_fwd_amd/csrc/fia_plan.cpp), with stand-ins for the device hooks,
under AddressSanitizer and UndefinedBehaviorSanitizer.  It mutates valid
configurations of every path (prefill, paged, decode, int8 KV, MLA,
block-sparse, FP8) with edge values (negative and huge dims, ranks 0 and 9,
unknown dtypes and layouts, NaN scales, INT64 extremes, length arrays of the
wrong count) and checks that every call returns a defined status, that a
failed phase 1 leaves no plan, and that accepted plans run.  Any out-of-bounds
read, signed overflow or leaked plan fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def fuzzer(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("fuzz") / "phase1_fuzz")
    cmd = [cxx, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "attention_fia_fwd_amd", "csrc"),
           os.path.join(ROOT, "tests", "phase1_fuzz.cpp"),
           os.path.join(ROOT, "attention_fia_fwd_amd", "csrc", "fia_plan.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if build.returncode != 0 and "sanitizer" in build.stderr.lower() and "cannot find" in build.stderr:
        pytest.skip("sanitizer runtime not installed")
    assert build.returncode == 0, build.stderr[-2000:]
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_phase1_random_inputs(fuzzer, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1")
    run = subprocess.run([fuzzer, "40000", str(seed)], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0 and run.stdout.strip().endswith("all ok"), \
        (run.stdout[-3000:] + run.stderr[-3000:])
