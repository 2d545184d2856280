// Issue schedule of the LDS reads of the d = 128 dK/dV kernel (plain C++,
// shared by the kernel and its host-side check).
#pragma once

namespace attn {
namespace bwd {

// Issue order of the LDS reads of one 32-row half of the d = 128 dK/dV
// kernel, so that every wait is exact.  A half starts with L row group 0, the
// 8 Q steps of S and the 4 row groups of -D in flight (reads 0 .. 12); then
// per slot: S phase slot ks reads the dP operands of step ks - (8 - PD) (dO,
// V block 0, V block 1); dP slot m reads the transposed dO of dV steps 0 / 1
// (m = 12 / 14), the dP operands of step m / 2 + PD (even m) and L group
// m / 4 + 1 (m = 0, 4, 8); dV slot m (even m) the transposed reads of dV step
// m / 2 + 2 or dK step m / 2 - 6; dK slot m (even, m < 12) the transposed Q
// of dK step m / 2 + 2.
struct W64Sched {
    static constexpr int KS = 8;
    static constexpr int PD = 4;                 // k steps of dP operands read ahead
    static constexpr int NH = 1 + KS + 4;        // reads at the start of a half
    static constexpr int S_LD(int ks) { return ks >= KS - PD ? 3 : 0; }
    static constexpr int P_TR(int m) { return (m == 12 || m == 14) ? 2 : 0; }
    static constexpr int P_DP(int m) { return (m % 2 == 0 && m / 2 + PD < KS) ? 3 : 0; }
    static constexpr int P_LV(int m) { return (m % 4 == 0 && m < 12) ? 1 : 0; }
    static constexpr int P_LD(int m) { return P_TR(m) + P_DP(m) + P_LV(m); }
    static constexpr int V_LD(int m) { return m % 2 == 0 ? 2 : 0; }
    static constexpr int K_LD(int m) { return (m % 2 == 0 && m / 2 + 2 < 8) ? 2 : 0; }
    // reads issued up to and including slot ks / m of each phase
    static constexpr int S_end(int ks) {
        int n = NH;
        for (int k = 0; k <= ks; ++k) n += S_LD(k);
        return n;
    }
    static constexpr int P_end(int m) {
        int n = S_end(KS - 1);
        for (int i = 0; i <= m; ++i) n += P_LD(i);
        return n;
    }
    static constexpr int V_end(int m) {
        int n = P_end(15);
        for (int i = 0; i <= m; ++i) n += V_LD(i);
        return n;
    }
    static constexpr int K_end(int m) {
        int n = V_end(15);
        for (int i = 0; i <= m; ++i) n += K_LD(i);
        return n;
    }
    // position of each read in the sequence (the later read of a pair)
    static constexpr int i_aq(int ks) { return 1 + ks; }
    static constexpr int i_lv(int rr) {
        return rr == 0 ? 0 : P_end(4 * (rr - 1) - 1) + P_TR(4 * (rr - 1)) + P_DP(4 * (rr - 1));
    }
    static constexpr int i_ado(int ks) {
        return ks < PD ? S_end(ks + KS - PD - 1) : P_end(2 * (ks - PD) - 1) + P_TR(2 * (ks - PD));
    }
    static constexpr int i_bv(int ks, int kb) { return i_ado(ks) + 1 + kb; }
    static constexpr int i_dd(int rr) { return 1 + KS + rr; }
    static constexpr int i_trv(int t) {
        return (t == 0 ? P_end(11) : t == 1 ? P_end(13) : V_end(2 * (t - 2) - 1)) + 1;
    }
    static constexpr int i_trk(int t) {
        return (t < 2 ? V_end(2 * (t + 6) - 1) : K_end(2 * (t - 2) - 1)) + 1;
    }
    // lgkmcnt of the wait before each slot's MFMA: every register is waited
    // for once, at the first slot that uses it (-1: no wait in that slot)
    static constexpr int mx(int a, int b) { return a > b ? a : b; }
    static constexpr int wait_S(int ks) { return S_end(ks - 1) - 1 - i_aq(ks); }
    static constexpr int wait_P(int m) {
        return (m & 1) ? P_end(m) - 1 - i_bv(m >> 1, 1)
               : m == 0 ? P_end(m) - 1 - mx(mx(i_bv(0, 0), i_lv(0)), i_dd(3))
               : (m & 3) == 0 ? P_end(m) - 1 - mx(i_bv(m >> 1, 0), i_lv(m >> 2))
                              : P_end(m) - 1 - i_bv(m >> 1, 0);
    }
    static constexpr int wait_V(int m) { return (m & 1) == 0 ? V_end(m) - 1 - i_trv(m >> 1) : -1; }
    static constexpr int wait_K(int m) { return (m & 1) == 0 ? K_end(m) - 1 - i_trk(m >> 1) : -1; }
};

}  // namespace bwd
}  // namespace attn
