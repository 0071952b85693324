"""The oracle's pins (tests/test_oracle.py) once more, with oracle.c built
under AddressSanitizer and UndefinedBehaviorSanitizer and loaded in its place
(host only): an out-of-bounds index or an overflow in the reference the GPU
path is checked against fails here instead of skewing the expected values."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_oracle_pins_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("sanitizer runtimes not installed")
    so = str(tmp_path / "liboracle_san.so")
    build = subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                            "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                            "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "oracle.c"),
                            "-o", so, "-lm"], capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-2000:]
    env = dict(os.environ, FIA_ORACLE_LIB=so, LD_PRELOAD=f"{asan} {ubsan}",
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0", OMP_NUM_THREADS="4")
    run = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle.py"),
                          "-x", "-q", "-p", "no:cacheprovider", "-p", "no:xdist"],
                         capture_output=True, text=True, timeout=1200, env=env, cwd=ROOT)
    assert run.returncode == 0, run.stdout[-3000:] + run.stderr[-3000:]
