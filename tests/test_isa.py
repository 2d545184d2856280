"""Compiled-code checks of the d = 128 dK/dV kernel and the dQ kernel (CPU only:
hipcc cross-compiles gfx950 without a GPU).

Both kernels issue LDS and global loads from inline assembly and wait for them
with explicit s_waitcnt counts, so the compiler does not know when a load's
destination registers are written.  A register copy that the compiler places
between such a load and its wait would read stale data.  These kernels are
written so that no copy of a vector register is ever needed; this test keeps it
that way across source and compiler changes by requiring every v_mov in them to
take an immediate or a scalar source.
"""
import os
import re
import shutil
import subprocess

import pytest

from exact_attention_bwd_amd import build as B

SRC = os.path.join(B.CSRC, "attn_bwd.hip")
KERNELS = (
    "_ZN4attn3bwd19bwd_dkdv_w64_kernelILb1E",
    "_ZN4attn3bwd19bwd_dkdv_w64_kernelILb0E",
    "_ZN4attn3bwd13bwd_dq_kernelILi128ELb1E",
    "_ZN4attn3bwd13bwd_dq_kernelILi128ELb0E",
    "_ZN4attn3bwd13bwd_dq_kernelILi64ELb1E",
    "_ZN4attn3bwd13bwd_dq_kernelILi64ELb0E",
)


@pytest.fixture(scope="module")
def isa(tmp_path_factory):
    hipcc = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("isa") / "attn_bwd.s")
    flags = [f for f in B.HIPCC_FLAGS if f != "-fPIC"]
    res = subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", SRC, "-o", out],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    with open(out) as f:
        return f.read().splitlines()


def _body(lines, prefix):
    start = next(i for i, l in enumerate(lines) if l.startswith(prefix) and l.split(":")[0].endswith("f"))
    end = next(i for i in range(start, len(lines)) if lines[i].startswith(".Lfunc_end"))
    return lines[start:end]


VMOV = re.compile(r"^\s*(v_mov_b32|v_mov_b64|v_pk_mov_b32)\S*\s+(\S+),\s*(.+)$")


@pytest.mark.parametrize("kernel", KERNELS)
def test_no_vector_register_copies(isa, kernel):
    body = _body(isa, kernel)
    assert any("v_mfma" in l for l in body), "kernel body not found"
    bad = []
    for l in body:
        m = VMOV.match(l)
        if m and re.match(r"v\[?\d", m.group(3).split(",")[0].strip()):
            bad.append(l.strip())
    assert not bad, f"{kernel}: vector register copies {bad[:5]}"
