"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): every library source is built with its device code as usual and
its host code instrumented, linked with a driver (tests/host_checks/) that
exercises validation, workspace sizes and layouts of the five workloads and of
thousands of random descriptors, and each entry point's argument checks; no
call reaches the GPU.  A sanitizer report or a failed check fails the test."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_code_under_sanitizers(tmp_path):
    script = os.path.join(ROOT, "tests", "host_checks", "build_and_run.sh")
    r = subprocess.run(["bash", script, str(tmp_path)], capture_output=True, text=True,
                       timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "host checks passed" in r.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
