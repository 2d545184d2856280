// Swizzled row-major LDS tiles and the direct global -> LDS copies that fill
// them (gfx950), shared by the attention kernels.
#pragma once

#include "common.hpp"

namespace attn {

// LDS tiles (all unpadded).  gfx950's LDS serves a 16-byte read for 16 lanes
// per clock across 64 banks, i.e. one 256-byte bank line.
//  * row-major [rows][HD] tiles (Q_i, dO_i, K_j, V_j): the 16-byte chunk c of
//    row r lives at chunk c ^ rswz<HD>(r).  For HD = 128 (one row per bank
//    line) rswz takes 16 distinct values on any 16 consecutive rows, so the
//    16-byte operand reads of 16 consecutive rows are conflict-free; its bits
//    2..3 are r & 3, so the 4 rows x 4 chunks of one transposing read also land
//    on 16 distinct chunks.  For HD = 64 (two rows per bank line) the same two
//    properties hold per row parity.
//  (The dQ kernel's dS tiles use a permutation of their own.)
template <int HD>
__device__ __forceinline__ int rswz(int r) {
    return HD == 128 ? (((r & 3) << 2) | ((r >> 2) & 3))
                     : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

template <int HD>
__device__ __forceinline__ int roff(int r, int c) {      // chunk c of row r (elements)
    return r * HD + ((c ^ rswz<HD>(r)) << 3);
}

template <int HD>
__device__ __forceinline__ int roff4(int r, int col) {   // 4 elements at col (multiple of 4)
    return r * HD + ((((col >> 3) ^ rswz<HD>(r))) << 3) + (col & 4);
}

// Copy ROWS rows of a [*, HD] bf16 tensor, starting at the descriptor's base,
// into a swizzled LDS tile with WAVES waves (rows past the descriptor's end
// arrive as zeros, whose contributions are masked).  voff[i] are the per-lane
// byte offsets of instruction i (see stage_offsets).
template <int HD, int ROWS, int WAVES>
__device__ __forceinline__ void stage_rows_b(__amdgpu_buffer_rsrc_t r, const int* voff, char* tile,
                                             int w) {
    constexpr int IPW = ROWS * (HD / 8) / 64 / WAVES;
#pragma unroll
    for (int i = 0; i < IPW; ++i) bdma16(r, voff[i], tile + (w * IPW + i) * 1024);
}

// Copy rows [row0, row0 + ROWS) of a [*, HD] bf16 tensor into a swizzled LDS
// tile with WAVES waves; rows at or past N re-read row N - 1 (finite values
// whose contributions are masked to zero).
template <int HD, int ROWS, int WAVES>
__device__ __forceinline__ void stage_rows(const __bf16* src, int row0, int N, char* tile, int w,
                                           int lane) {
    constexpr int CPR = HD / 8;
    constexpr int IPW = ROWS * CPR / 64 / WAVES;          // instructions per wave
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int I = w * IPW + i;
        const int P = I * 64 + lane;                       // physical chunk
        const int r = P / CPR;
        const int c = (P % CPR) ^ rswz<HD>(r);             // logical chunk stored there
        const int row = min(row0 + r, N - 1);
        dma16(src + (size_t)row * HD + c * 8, tile + I * 1024);
    }
}

// Per-lane source byte offsets for stage_rows_b: the physical chunk this lane
// writes belongs to row r, logical chunk (p ^ rswz(r)).
template <int HD, int ROWS, int WAVES>
__device__ __forceinline__ void stage_offsets(int* voff, int w, int lane) {
    constexpr int CPR = HD / 8;
    constexpr int IPW = ROWS * CPR / 64 / WAVES;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int P = (w * IPW + i) * 64 + lane;
        const int r = P / CPR;
        voff[i] = (r * HD + (((P % CPR) ^ rswz<HD>(r)) << 3)) * 2;
    }
}

// Copy BYTES contiguous bytes (a multiple of WAVES * 1024) into LDS.
template <int BYTES, int WAVES>
__device__ __forceinline__ void stage_bytes(const char* src, char* dst, int w, int lane) {
    constexpr int IPW = BYTES / 1024 / WAVES;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int I = w * IPW + i;
        dma16(src + I * 1024 + lane * 16, dst + I * 1024);
    }
}

}  // namespace attn
