"""Host-side pieces of bench.py: the code key that ties a committed HBM-traffic
profile to the GEMM code it was measured on (CPU only)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_key_ignores_comments_but_not_code(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("int f(int x) {  // add one\n  return x + 1;\n}\n")
    b = tmp_path / "b.hip"
    b.write_text("// a new header line\nint f(int x) {  // adds one\n\n  return x + 1;   \n}\n")
    c = tmp_path / "c.hip"
    c.write_text("int f(int x) {  // add one\n  return x + 2;\n}\n")
    assert bench.code_sha256(str(a)) == bench.code_sha256(str(b))
    assert bench.code_sha256(str(a)) != bench.code_sha256(str(c))


def test_committed_traffic_profile_matches_the_gemm_code():
    # the skewed layer's up-GEMM counters were taken on the code as it stands
    t = bench.traffic_from_profile("zipf_skew_bf16", "up")
    assert t is not None and t > 0
    assert bench.traffic_from_profile("no_such_workload", "up") is None


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_host_cpu_record_names_the_cpus_seen():
    h = bench._host_cpu()
    assert h["logical_cpus_visible"] >= 1
    assert h["cpu_model"] is None or isinstance(h["cpu_model"], str)
