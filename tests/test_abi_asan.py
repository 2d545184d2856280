"""The C entry points' argument validation, built for the host only with
AddressSanitizer (no GPU, no kernels: the launchers are stand-ins that record
being reached).  Every invalid argument must return its documented status
without reaching a launcher, every valid call must reach one, and the
sanitizer must report nothing (message formatting, pointer checks)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_validation_paths_under_asan(tmp_path):
    hipcc = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "validate")
    srcs = [os.path.join(ROOT, "exact_attention_bwd_amd", "csrc", "attn_api.hip"),
            os.path.join(ROOT, "tests", "asan", "launch_stub.cpp"),
            os.path.join(ROOT, "tests", "asan", "validate_main.cpp")]
    # host-only build; the sanitizer applies to the host pass only
    cmd = [hipcc, "-x", "hip", "--offload-host-only", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", *srcs, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0 and run.stdout.strip().startswith("ok"), run.stdout[-3000:] + run.stderr[-3000:]
    assert "AddressSanitizer" not in run.stderr, run.stderr[-3000:]
