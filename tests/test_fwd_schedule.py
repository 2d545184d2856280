"""Host check of the LDS-read schedule of the d = 128 forward kernel (CPU only).

Per key tile a wave of the kernel reads 32 matrix-core operands from LDS:
16 K-row operands (one ds_read_b128 each) for S^T = K Q^T, then 16 V^T
operands (two ds_read_b64_tr_b16 each) for O^T += V^T P^T.  At need point n
it issues operand n + D (past 31: the next tile's K rows) and then waits for
operand n with the lgkmcnt that FwdSched (csrc/fwd_sched.hpp) computes.  LDS
operations complete in order, so the count is right exactly when it equals the
number of LDS instructions issued after the awaited operand.  This test
compiles the header with the host compiler and compares its counts with a
simulation of the issue order written out here:

  * prologue (K rows of tile 0 only): operands 0 .. D - 1 are issued up front,
    need point n (0 .. 15) issues operand n + D while that is a K operand;
  * steady state: operands 0 .. D - 1 of the tile were issued at the end of
    the previous iteration; need point n (0 .. 31) issues operand n + D, where
    32 + j stands for K operand j of the next iteration.
"""
import shutil
import subprocess

import pytest

from exact_attention_bwd_amd import build as B

PROG = r"""
#include <cstdio>
#include "fwd_sched.hpp"
using S = attn::fwd::FwdSched;
int main() {
    std::printf("D %d B %d\n", S::D, S::BARRIER_N);
    for (int n = 0; n < 16; ++n) std::printf("P %d %d %d\n", n, (int)S::issues(S::PRO, n), S::wait(S::PRO, n));
    for (int n = 0; n < 32; ++n) std::printf("I %d %d %d\n", n, (int)S::issues(S::ITER, n), S::wait(S::ITER, n));
    return 0;
}
"""


@pytest.fixture(scope="module")
def sched(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("fsched")
    src, exe = d / "s.cpp", d / "s"
    src.write_text(PROG)
    subprocess.run([cxx, "-std=c++17", "-I", B.CSRC, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    head = out[0].split()
    got = {}
    for line in out[1:]:
        if line:
            m, n, iss, w = line.split()
            got[(m, int(n))] = (bool(int(iss)), int(w))
    return int(head[1]), int(head[3]), got


def n_inst(j):
    return 1 if j % 32 < 16 else 2


def simulate(D, prologue):
    """Wait count needed at each need point, from the instruction stream."""
    seq = []
    for j in range(D):
        seq += [j] * n_inst(j)
    need, issued = {}, {}
    for n in range(16 if prologue else 32):
        j = n + D
        issued[n] = j < 16 if prologue else True
        if issued[n]:
            seq += [j] * n_inst(j)
        last = max(i for i, x in enumerate(seq) if x == n)
        need[n] = len(seq) - 1 - last
    return need, issued


def test_prologue_waits(sched):
    D, _, got = sched
    need, issued = simulate(D, True)
    bad = {n: (got[("P", n)], (issued[n], need[n])) for n in need if got[("P", n)] != (issued[n], need[n])}
    assert not bad, bad


def test_steady_state_waits(sched):
    D, _, got = sched
    need, issued = simulate(D, False)
    bad = {n: (got[("I", n)], (issued[n], need[n])) for n in need if got[("I", n)] != (issued[n], need[n])}
    assert not bad, bad
    assert max(need.values()) <= 15, "lgkmcnt holds 0 .. 15"


def test_barrier_precedes_next_tile_reads(sched):
    """The barrier (which makes the next tile's K copy visible) sits at the
    first need point that issues a next-iteration operand."""
    D, barrier, _ = sched
    first = min(n for n in range(32) if n + D >= 32)
    assert barrier == first
    assert 16 <= barrier < 32, "the barrier falls in the PV phase, after the K reads of the tile"
