"""bench.py's host-side contract (no GPU): it refuses more than one GPU with a
message and exit status 2 before touching a device, its options parse, and
roofline.traffic comes from the committed counter summary only while that
summary names the sha256 of the kernel source being run."""
import hashlib
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""


def test_help_lists_the_workloads():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0
    for w in ("c1", "c3", "c4", "c5", "paged_prefill", "mtp_decode", "int8_decode",
              "int8_paged_decode", "fp8_bsa", "mla_decode", "mla_shared_kv"):
        assert w in r.stdout


def test_traffic_only_for_the_profiled_kernel_source(tmp_path, monkeypatch):
    src = os.path.join(ROOT, "attention_fia_fwd_amd", "csrc", "fia_kernels.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    summary = open(os.path.join(ROOT, "profiles", "hbm_traffic_counters.txt")).read()
    committed = dict(l.strip().split("=", 1) for l in summary.splitlines() if "=" in l and not l.startswith("#"))
    t = bench.measured_traffic("c2")
    if committed["kernel_source_sha256_prefix"] == sha:
        assert isinstance(t, int) and t > 0
    else:
        assert t is None
    # a summary of another source gives None, one of this source the scaled bytes
    prof = tmp_path / "profiles"
    prof.mkdir()
    (tmp_path / "attention_fia_fwd_amd" / "csrc").mkdir(parents=True)
    (tmp_path / "attention_fia_fwd_amd" / "csrc" / "fia_kernels.hip").write_bytes(open(src, "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    body = "fetch_scale=2.0\nwrite_scale=1.0\nc2_fetch_kib=100\nc2_write_kib=50\n"
    (prof / "hbm_traffic_counters.txt").write_text(f"kernel_source_sha256_prefix={'0' * 16}\n" + body)
    assert bench.measured_traffic("c2") is None
    (prof / "hbm_traffic_counters.txt").write_text(f"kernel_source_sha256_prefix={sha}\n" + body)
    assert bench.measured_traffic("c2") == 100 * 1024 * 2 + 50 * 1024
    assert bench.measured_traffic("c3") is None
