// LDS-read schedule of the d = 128 forward kernel (fwd_w64_kernel), as
// compile-time functions so that the host can check them.
//
// Per key tile a wave reads 32 matrix-core operands from LDS, in this order
// (one "stream" per iteration):
//   operand j = 0 .. 15   K rows: key block j / 8, head-dim step j % 8
//                         (one ds_read_b128 each), for S^T = K Q^T
//   operand j = 16 .. 31  V^T: v = j - 16, head-dim block v % 4, key step
//                         v / 4 (two ds_read_b64_tr_b16 each), for O^T += V^T P^T
// Operand j is needed at "need point" j: the S phase of an iteration has need
// points 0 .. 15 (two MFMAs each), the PV phase 16 .. 31.  At need point n the
// wave first issues operand n + D, then waits for operand n; LDS operations
// complete in order, so lgkmcnt(count) with count = the number of LDS
// instructions issued after operand n suffices.  Operands past 31 belong to
// the next iteration (its K rows, read from the other K slot once the
// barrier at need point 32 - D has made them visible).
#pragma once

namespace attn {
namespace fwd {

struct FwdSched {
    static constexpr int D = 3;                  // operands in flight
    static constexpr int NOPS = 32;              // operands per iteration
    static constexpr int NK = 16;                // of which K rows
    // stream modes
    static constexpr int PRO = 0;                // prologue S phase: K rows of tile 0 only
    static constexpr int ITER = 1;               // steady state: issues wrap into the next iteration

    static constexpr int inst(int j) { return (j % NOPS) < NK ? 1 : 2; }
    static constexpr int limit(int mode) { return mode == PRO ? NK - 1 : NOPS - 1 + D; }
    // does need point n issue operand n + D?
    static constexpr bool issues(int mode, int n) { return n + D <= limit(mode); }
    // lgkmcnt for the wait at need point n
    static constexpr int wait(int mode, int n) {
        int c = 0;
        const int hi = n + D < limit(mode) ? n + D : limit(mode);
        for (int j = n + 1; j <= hi; ++j) c += inst(j);
        return c;
    }
    // need point at which the barrier (and the next copies) go: just before
    // the first issue of a next-iteration operand
    static constexpr int BARRIER_N = NOPS - D;
};

}  // namespace fwd
}  // namespace attn
