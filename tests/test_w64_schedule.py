"""Host check of the LDS-read schedule of the d = 128 dK/dV kernel (CPU only).

The kernel issues every LDS read of a 32-row half from assembly and waits for
each with an explicit lgkmcnt that W64Sched (csrc/w64_sched.hpp) derives from
the issue order.  LDS reads complete in order, so the count is right exactly
when it equals the number of reads issued after the awaited one.  This test
compiles the header with the host compiler, prints the counts, and compares
them with a slot-by-slot simulation of the kernel's issue order written out
here independently:

  * a half starts with L group 0, the 8 Q operands of S and the 4 row groups
    of -D (the dP accumulators' initial value) in flight;
  * S slot ks: wait for Q step ks, then (ks >= 8 - PD) read the dP operands
    of step ks - (8 - PD): dO, V block 0, V block 1;
  * dP slot m: transposed dO of dV step 0 / 1 (m = 12 / 14), the dP operands
    of step m / 2 + PD (even m), L group m / 4 + 1 (m = 0, 4, 8), then the
    wait for this slot's operands (slot 0 also for -D);
  * dV slot m: (even m) the transposed reads of dV step m / 2 + 2, or of dK
    step m / 2 - 6 once those run out;
  * dK slot m: (even m, m < 12) transposed Q of dK step m / 2 + 2.
"""
import os
import shutil
import subprocess

import pytest

from exact_attention_bwd_amd import build as B

PROG = r"""
#include <cstdio>
#include "w64_sched.hpp"
using S = attn::bwd::W64Sched;
int main() {
    std::printf("PD %d\n", S::PD);
    for (int k = 0; k < 8; ++k) std::printf("S %d %d\n", k, S::wait_S(k));
    for (int m = 0; m < 16; ++m) std::printf("P %d %d\n", m, S::wait_P(m));
    for (int m = 0; m < 16; ++m) std::printf("V %d %d\n", m, S::wait_V(m));
    for (int m = 0; m < 16; ++m) std::printf("K %d %d\n", m, S::wait_K(m));
    return 0;
}
"""


@pytest.fixture(scope="module")
def waits(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("sched")
    src, exe = d / "sched.cpp", d / "sched"
    src.write_text(PROG)
    subprocess.run([cxx, "-std=c++17", "-I", B.CSRC, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {}
    pd = None
    for line in out:
        if not line:
            continue
        f = line.split()
        if f[0] == "PD":
            pd = int(f[1])
        else:
            got[(f[0], int(f[1]))] = int(f[2])
    return pd, got


def simulate(pd):
    seq = ["lv0"] + [f"aq{k}" for k in range(8)] + [f"dd{r}" for r in range(4)]
    need = {}

    def wait(tag, names):
        idx = max(seq.index(n) for n in names)
        need[tag] = len(seq) - 1 - idx

    def load_dp(k):
        seq.extend([f"ado{k}", f"bv{k}_0", f"bv{k}_1"])

    for ks in range(8):
        wait(("S", ks), [f"aq{ks}"])
        if ks >= 8 - pd:
            load_dp(ks - (8 - pd))
    for m in range(16):
        ks, kb, rr = m >> 1, m & 1, m >> 2
        if m in (12, 14):
            t = (m - 12) // 2
            seq.extend([f"trv{t}a", f"trv{t}b"])
        if kb == 0 and ks + pd < 8:
            load_dp(ks + pd)
        if m % 4 == 0 and m < 12:
            seq.append(f"lv{rr + 1}")
        if m == 0:
            wait(("P", m), ["ado0", "bv0_0", "lv0", "dd0", "dd1", "dd2", "dd3"])
        elif kb == 1:
            wait(("P", m), [f"bv{ks}_1"])
        elif m % 4 == 0:
            wait(("P", m), [f"ado{ks}", f"bv{ks}_0", f"lv{rr}"])
        else:
            wait(("P", m), [f"ado{ks}", f"bv{ks}_0"])
    for m in range(16):
        t, kb = m >> 1, m & 1
        if kb == 0:
            if t + 2 < 8:
                seq.extend([f"trv{t + 2}a", f"trv{t + 2}b"])
            else:
                seq.extend([f"trk{t - 6}a", f"trk{t - 6}b"])
        if kb == 0:
            wait(("V", m), [f"trv{t}a", f"trv{t}b"])
        else:
            need[("V", m)] = -1
    for m in range(16):
        t = m >> 1
        if m % 2 == 0 and t + 2 < 8:
            seq.extend([f"trk{t + 2}a", f"trk{t + 2}b"])
        if m % 2 == 0:
            wait(("K", m), [f"trk{t}a", f"trk{t}b"])
        else:
            need[("K", m)] = -1
    return need, seq


def test_waits_match_issue_order(waits):
    pd, got = waits
    assert 1 <= pd <= 8
    need, seq = simulate(pd)
    # L 0, Q x 8, -D 0..3, dP operands 8 x 3, L 1..3, transposed pairs 16 x 2
    assert len(seq) == 9 + 8 * 3 + 3 + 4 + 16 * 2, "every LDS read of a half issued exactly once"
    assert len(set(seq)) == len(seq)
    bad = {k: (got[k], v) for k, v in need.items() if got[k] != v}
    assert not bad, f"wait counts differ from the issue order (got, needed): {bad}"


def test_waits_fit_the_counter(waits):
    """lgkmcnt holds 0..15; larger counts are clamped to 15 in the kernel,
    which only waits longer.  A negative count would mean a read is used
    before it is issued."""
    _, got = waits
    assert all(v >= -1 for v in got.values())
    assert all(v >= 0 for (ph, _), v in got.items() if ph in ("S", "P"))
