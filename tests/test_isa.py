"""Compiled-code checks of the hand-scheduled kernels: the d = 128 dK/dV kernel,
the dQ kernel and the d = 128 forward kernel (CPU only: hipcc cross-compiles
gfx950 without a GPU).

These kernels issue LDS and global loads from inline assembly and wait for them
with explicit s_waitcnt counts, so the compiler does not know when a load's
destination registers are written.  A register copy that the compiler places
between such a load and its wait would read stale data.  The kernels are
written so that the compiler never needs to copy a vector register; this test
keeps it that way across source and compiler changes by requiring every
compiler-generated v_mov in them to take an immediate or a scalar source
(copies written inside the kernels' own assembly blocks are deliberate and
exempt), and by requiring that they spill nothing.
"""
import os
import re
import shutil
import subprocess

import pytest

from exact_attention_bwd_amd import build as B

KERNELS = (
    ("attn_bwd.hip", "_ZN4attn3bwd19bwd_dkdv_w64_kernelILb1E"),
    ("attn_bwd.hip", "_ZN4attn3bwd19bwd_dkdv_w64_kernelILb0E"),
    ("attn_bwd.hip", "_ZN4attn3bwd13bwd_dq_kernelILi128ELb1E"),
    ("attn_bwd.hip", "_ZN4attn3bwd13bwd_dq_kernelILi128ELb0E"),
    ("attn_bwd.hip", "_ZN4attn3bwd13bwd_dq_kernelILi64ELb1E"),
    ("attn_bwd.hip", "_ZN4attn3bwd13bwd_dq_kernelILi64ELb0E"),
    ("attn_fwd.hip", "_ZN4attn3fwd14fwd_w64_kernelILb1ELi1E"),
    ("attn_fwd.hip", "_ZN4attn3fwd14fwd_w64_kernelILb0ELi1E"),
)


@pytest.fixture(scope="module")
def isa(tmp_path_factory):
    hipcc = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    flags = [f for f in B.HIPCC_FLAGS if f != "-fPIC"]
    out = {}
    d = tmp_path_factory.mktemp("isa")
    for src in sorted({s for s, _ in KERNELS}):
        asm = str(d / (src + ".s"))
        res = subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", asm],
                             capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        with open(asm) as f:
            out[src] = f.read().splitlines()
    return out


def _body(lines, prefix):
    start = next(i for i, l in enumerate(lines) if l.startswith(prefix) and l.split(":")[0].endswith("f"))
    end = next(i for i in range(start, len(lines)) if lines[i].startswith(".Lfunc_end"))
    return lines[start:end]


VMOV = re.compile(r"^\s*(v_mov_b32|v_mov_b64|v_pk_mov_b32)\S*\s+(\S+),\s*(.+)$")


def _compiler_lines(body):
    """The kernel's instructions outside its inline-assembly blocks."""
    inside = False
    for l in body:
        if "ASMSTART" in l:
            inside = True
        elif "ASMEND" in l:
            inside = False
        elif not inside:
            yield l


@pytest.mark.parametrize("src,kernel", KERNELS, ids=[k for _, k in KERNELS])
def test_no_vector_register_copies(isa, src, kernel):
    body = _body(isa[src], kernel)
    assert any("v_mfma" in l for l in body), "kernel body not found"
    bad = []
    for l in _compiler_lines(body):
        m = VMOV.match(l)
        if m and re.match(r"v\[?\d", m.group(3).split(",")[0].strip()):
            bad.append(l.strip())
    assert not bad, f"{kernel}: vector register copies {bad[:5]}"


@pytest.mark.parametrize("src,kernel", KERNELS, ids=[k for _, k in KERNELS])
def test_no_spills(isa, src, kernel):
    lines = isa[src]
    meta = next(i for i, l in enumerate(lines) if l.strip().startswith(".name:") and l.split()[-1].startswith(kernel))
    # the kernel's metadata entry: spill counters follow its .name
    end = next((i for i in range(meta + 1, len(lines)) if lines[i].strip().startswith((".name:", "- .", "..."))), len(lines))
    spills = [int(l.split()[-1]) for l in lines[meta:end] if l.strip().startswith((".vgpr_spill_count:", ".sgpr_spill_count:"))]
    assert spills and max(spills) == 0, f"{kernel}: spills {spills}"
