"""Compiled-code checks of the hand-scheduled kernels: the d = 128 dK/dV kernel,
the dQ kernel and the d = 128 forward kernel (CPU only: hipcc cross-compiles
gfx950 without a GPU).

These kernels issue LDS and global loads and matrix-core products from inline
assembly and wait for them with explicit s_waitcnt counts and s_nop settles,
so the compiler knows neither when a load's destination registers are written
nor when a product's result lands.  A register copy that the compiler places
between such an instruction and its wait or settle would read stale data.
The kernels are written so that no such copy is needed; this test keeps it
that way across source and compiler changes:

- every compiler-generated v_mov takes an immediate, a scalar, or a register
  that holds only an immediate (a zero fill) as its source;
- no compiler move reads an AGPR that the kernel's assembly writes while
  products are still being issued;
- after the last product, no compiler move reads that product's result
  before the settle that follows it;
- and the kernels spill nothing.

The fused backward's sweep kernel runs an item behind a call
(fused_item_call): a call saves and restores the callee-saved registers
through scratch, and the allocator copies a few of its own values.  For it
the rule is the hazard itself: no compiler copy or scratch store reads a
register that the function's assembly wrote last.  (The sweep kernel only
takes tickets that no workgroup of their XCD took, which normally never
happens; its speed does not matter.)

Copies inside the kernels' own assembly blocks are deliberate and exempt.
"""
import os
import re
import shutil
import subprocess

import pytest

from exact_attention_bwd_amd import build as B

KERNELS = (
    ("attn_bwd.hip", "_ZN4attn3bwd16bwd_fused_kernelILb0E"),
    ("attn_bwd.hip", "_ZN4attn3bwd16bwd_fused_kernelILb1E"),
    ("attn_bwd.hip", "_ZN4attn3bwd15fused_item_callILb0E"),
    ("attn_bwd.hip", "_ZN4attn3bwd15fused_item_callILb1E"),
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
    start = next(i for i, l in enumerate(lines) if l.startswith(prefix) and l.split(";")[0].rstrip().endswith(":"))
    end = next(i for i in range(start, len(lines)) if lines[i].startswith(".Lfunc_end"))
    return lines[start:end]


VMOV = re.compile(r"^\s*(v_mov_b32|v_mov_b64|v_pk_mov_b32|v_accvgpr_mov_b32|v_accvgpr_read_b32|v_accvgpr_write_b32)\S*\s+(\S+),\s*(.+)$")


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


REG = re.compile(r"([va])\[?(\d+)(?::(\d+))?\]?$")


def _regs(op):
    """Registers named by an operand ('v5', 'a[16:19]'), as {('a', 16), ...}."""
    m = REG.match(op.strip())
    if not m:
        return set()
    lo = int(m.group(2))
    return {(m.group(1), r) for r in range(lo, int(m.group(3) or lo) + 1)}


STORE = re.compile(r"^\s*(ds_write|buffer_store|global_store|flat_store|scratch_store|s_)")
IMM = re.compile(r"^-?(0x[0-9a-f]+|\d+(\.\d+)?)$")


FUNCTIONS = ("_ZN4attn3bwd15fused_item_callILb0E", "_ZN4attn3bwd15fused_item_callILb1E")


@pytest.mark.parametrize("src,kernel", KERNELS, ids=[k for _, k in KERNELS])
def test_no_vector_register_copies(isa, src, kernel):
    body = _body(isa[src], kernel)
    assert any("v_mfma" in l for l in body), "kernel body not found"
    # the products issued from assembly (their latency is unknown to the
    # compiler); a kernel whose products are all compiler-issued: all of them
    in_asm, asm_mfma = False, []
    for i, l in enumerate(body):
        if "ASMSTART" in l:
            in_asm = True
        elif "ASMEND" in l:
            in_asm = False
        elif in_asm and "v_mfma" in l:
            asm_mfma.append(i)
    mfma = asm_mfma or [i for i, l in enumerate(body) if "v_mfma" in l]
    first, last = mfma[0], mfma[-1]
    settle = next((i for i in range(last, len(body)) if "s_nop 15" in body[i]), len(body))
    # registers the kernels' own assembly writes (loads, products): the
    # compiler knows neither when they land nor the products' latency
    asm_dst, inside, asm_lines = set(), False, set()
    for i, l in enumerate(body):
        if "ASMSTART" in l:
            inside = True
        elif "ASMEND" in l:
            inside = False
        elif inside and l.strip() and not STORE.match(l):
            asm_lines.add(i)
            parts = l.split(None, 1)
            if len(parts) > 1:
                asm_dst |= _regs(parts[1].split(",")[0])
    last_dst = _regs(body[last].split()[1].rstrip(",")) if last in asm_lines else set()
    # registers that every write in the body sets to an immediate: constants
    # wherever they are read (a zero the compiler keeps for accumulator fills
    # outside a loop, say)
    imm_w, other_w = set(), set()
    for l in body:
        parts = l.split(None, 1)
        if len(parts) < 2 or STORE.match(l) or not l.startswith(("\tv_", "\ts_", "\tds_", "\tbuffer", "\tglobal")):
            continue
        dst = _regs(parts[1].split(",")[0])
        m = VMOV.match(l)
        if m and IMM.match(m.group(3).split(",")[0].strip()):
            imm_w |= dst
        else:
            other_w |= dst
    fixed = imm_w - other_w
    bad = []
    inside = False
    const = set(fixed)     # registers whose latest value is an immediate (zero fills)
    last_asm = {}          # register -> whether its latest writer (in program text) is assembly
    for i, l in enumerate(body):
        if "ASMSTART" in l:
            inside = True
            continue
        if "ASMEND" in l:
            inside = False
            continue
        if l.strip() and not STORE.match(l) and len(l.split(None, 1)) > 1:
            for r in _regs(l.split(None, 1)[1].split(",")[0]):
                last_asm[r] = inside
        if re.match(r"^\.LBB\S*:", l):
            const = set(fixed)                   # a block may be reached from elsewhere
            continue
        parts = l.split(None, 1)
        dst = _regs(parts[1].split(",")[0]) if len(parts) > 1 and not STORE.match(l) else set()
        m = None if inside else VMOV.match(l)
        if m is None:
            const -= dst
            continue
        src_op = m.group(3).split(",")[0].strip()
        srcs = _regs(src_op)
        if IMM.match(src_op) or (srcs and srcs <= const):
            const |= dst                         # an immediate, or a copy of one
            continue
        const -= dst
        if not srcs:
            continue                             # scalar source
        from_v = any(k == "v" for k, _ in srcs)
        if m.group(1).startswith("v_mov") or m.group(1) == "v_pk_mov_b32":
            # a copy of a VGPR that assembly fills somewhere in the body
            # (functions: whose latest writer is assembly); copies of values
            # the compiler computed itself (a loop's hoisted bases) are safe
            if from_v and (srcs & asm_dst if kernel not in FUNCTIONS else any(last_asm.get(r) for r in srcs)):
                bad.append(l.strip())
        elif first <= i < last and srcs & asm_dst:
            bad.append(l.strip())                # AGPR traffic among the products
        elif last <= i < settle and srcs & last_dst:
            bad.append(l.strip())                # the last product read before its settle
    assert not bad, f"{kernel}: vector register copies {bad[:5]}"


@pytest.mark.parametrize("src,kernel", [k for k in KERNELS if k[1] in FUNCTIONS], ids=lambda k: str(k))
def test_function_spills_are_not_of_pending_registers(isa, src, kernel):
    body = _body(isa[src], kernel)
    scratch = [i for i, l in enumerate(body) if "scratch_" in l]
    # the callee-saved registers are saved before the first assembly block
    # and restored after the last one; in between, no scratch store may
    # write out a register whose latest writer (in program text) is the
    # functions' assembly (its load or product may not have landed)
    first = next(i for i, l in enumerate(body) if "ASMSTART" in l)
    last = max(i for i, l in enumerate(body) if "ASMEND" in l)
    last_asm, inside, bad = {}, False, []
    for i, l in enumerate(body):
        if "ASMSTART" in l:
            inside = True
            continue
        if "ASMEND" in l:
            inside = False
            continue
        parts = l.split(None, 1)
        if "scratch_store" in l and first < i < last:
            if any(last_asm.get(r) for r in _regs(parts[1].split(",")[1])):
                bad.append(l.strip())
        elif l.strip() and not STORE.match(l) and len(parts) > 1:
            for r in _regs(parts[1].split(",")[0]):
                last_asm[r] = inside
    assert not bad, f"{kernel}: spills of registers the assembly wrote last {bad[:5]}"


@pytest.mark.parametrize("src,kernel", [k for k in KERNELS if k[1] not in FUNCTIONS], ids=lambda k: str(k))
def test_no_spills(isa, src, kernel):
    """No vector register spills (scratch memory) anywhere.  Scalar registers
    spilled into lanes of a vector register (no memory traffic) are allowed
    only where their reloads stay out of nested loops: the persistent fused
    kernel holds its arguments across the item loop and reloads some of them
    once per item, never inside the tile loop."""
    lines = isa[src]
    meta = next(i for i, l in enumerate(lines) if l.strip().startswith(".name:") and l.split()[-1].startswith(kernel))
    # the kernel's metadata entry: spill counters follow its .name
    end = next((i for i in range(meta + 1, len(lines)) if lines[i].strip().startswith((".name:", "- .", "..."))), len(lines))
    counts = {l.split()[0].rstrip(":"): int(l.split()[-1]) for l in lines[meta:end]
              if l.strip().startswith((".vgpr_spill_count:", ".sgpr_spill_count:"))}
    assert len(counts) == 2, counts
    assert counts[".vgpr_spill_count"] == 0, f"{kernel}: {counts}"
    if counts[".sgpr_spill_count"]:
        depth, nested = 0, []
        for l in _body(lines, kernel):
            m = re.search(r"Depth=(\d+)", l)
            if re.match(r"^\.LBB\S*:", l) or l.startswith("; %bb"):
                depth = int(m.group(1)) if m else 0
            if "v_readlane" in l and depth >= 2:
                nested.append(l.strip())
        assert not nested, f"{kernel}: {counts}, reloads in nested loops {nested[:3]}"


@pytest.mark.parametrize("src,kernel", KERNELS, ids=[k for _, k in KERNELS])
def test_no_scalar_loads_among_counted_lds_reads(isa, src, kernel):
    """The kernels wait for their LDS reads with exact lgkmcnt counts, which
    assume that only LDS reads are counted: a scalar memory load (also
    counted by lgkmcnt, and completing out of order) between the first and
    the last of those reads would make a wait end early."""
    body = _body(isa[src], kernel)
    inside, reads = False, []
    for i, l in enumerate(body):
        if "ASMSTART" in l:
            inside = True
        elif "ASMEND" in l:
            inside = False
        elif inside and l.strip().startswith("ds_read"):
            reads.append(i)
    assert reads, "no counted LDS reads found"
    smem = [body[i].strip() for i in range(reads[0], reads[-1])
            if body[i].strip().startswith(("s_load", "s_buffer_load", "s_scratch_load", "s_memtime", "s_memrealtime"))]
    assert not smem, f"{kernel}: scalar loads among the counted LDS reads {smem[:3]}"
