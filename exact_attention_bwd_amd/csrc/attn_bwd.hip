// Exact attention backward for gfx950: the preprocess D = rowsum(dO o O), a
// small row-statistics prep, the dK/dV kernel (which also stores dS) and the
// dQ kernel.
//
// The method is the tiled backward of "Writing Speed-of-Light Attention
// Backward Kernel for 5090 in CUDA" (hoanh.space): sections "Precomputing D",
// "Main backward kernel" and the tiled-backward pseudocode after
// "Mathematical Formulation".  One workgroup owns one key/value tile K_j, V_j
// of one (batch, head), keeps dK_j and dV_j in registers, walks the query
// tiles i (from the diagonal tile when causal) and recomputes S_ij and P_ij
// from the saved log-sum-exp L.
//
// dQ: the page adds every column block's dQ_i partial into an fp32 buffer with
// atomics.  On this GPU fp32 atomics to device memory are executed at the
// memory side and sustain about 1.35 TB/s, against 6.8 TB/s for plain stores,
// and the causal 8x16x4096x128 problem would need 4.4 GB of them.  Instead
// the dK/dV kernel writes each dS_ij (bf16, the same rounding the page applies
// before its dQ product) to a workspace tile, and a second, query-parallel
// kernel forms dQ_i = scale * sum_j dS_ij K_j in fp32 registers.  The kernel
// boundary is the grid-wide synchronisation; nothing is accumulated out of
// order, so the results are bitwise reproducible.
//
// CDNA4 mapping (not the page's SM120 one):
//  * dK/dV kernel for d = 128 (bwd_dkdv_w64_kernel): 4 wave64s, one per SIMD,
//    per 256-key tile; each wave owns 64 keys and every query row, keeps K in
//    registers and dK / dV in the accumulation registers.
//  * dK/dV kernel for other d (bwd_dkdv_kernel): 512 threads = 8 wave64s (two
//    per SIMD).  The workgroup owns B_c = 128 keys; wave (kw, qh) owns keys
//    32 kw .. + 31 and query rows 32 qh .. + 31 of each 64-row query tile.
//  * S = Q K^T and dP = dO V^T take both operands from LDS.  Their accumulator
//    layout (one key per lane) is exactly the A layout of P^T and dS^T, so
//    dV = P^T dO and dK = dS^T Q take P and dS straight from registers, with
//    the query index relabelled consistently on the B side (dO and Q read
//    with transposing LDS reads).
//  * Q_i / dO_i tiles are double-buffered in LDS by direct buffer -> LDS
//    copies issued one tile ahead; all LDS tiles are XOR-swizzled for the
//    64-bank LDS.
//  * P = exp(scale * S - L) is evaluated as 2^(S * scale * log2 e - L * log2 e)
//    with v_exp_f32.
//  * dQ kernel: 4 wave64s per (batch*head, 64-row query tile); dS tiles are
//    copied into an LDS double buffer and read transposed, K comes from a
//    register-ready image of K_j that the dK/dV kernel writes once per tile.
#include <type_traits>

#include "asm_ops.hpp"
#include "common.hpp"
#include "launch.hpp"
#include "tiles.hpp"
#include "w64_sched.hpp"

namespace attn {

// ----------------------------------------------------------------------------
// D = rowsum(dO o O) in fp32 ("Precomputing D").  HD / 8 lanes share one row,
// each loads 16 bytes of O and dO; the partial sums are combined by lane
// exchanges inside the group.  Grid-stride over rows.
// ----------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(
    const __bf16* __restrict__ O, const __bf16* __restrict__ dO, float* __restrict__ D,
    long long rows) {
    constexpr int LPR = HD / 8;                 // lanes per row
    constexpr int RPB = 256 / LPR;              // rows per block pass
    const int t = threadIdx.x;
    const int sub = t % LPR;
    for (long long row = (long long)blockIdx.x * RPB + t / LPR; row < rows;
         row += (long long)gridDim.x * RPB) {
        const size_t off = (size_t)row * HD + sub * 8;
        const bf16x8 o = *reinterpret_cast<const bf16x8*>(O + off);
        const bf16x8 g = *reinterpret_cast<const bf16x8*>(dO + off);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += (float)o[e] * (float)g[e];
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
        if (sub == 0) D[row] = acc;
    }
}

// Backward prep: the per-row statistics the dK/dV kernel copies into LDS,
// padded to the 64-row query tile: Lb = L * log2(e) (+inf past the end, so
// P = 2^-inf = 0 there) and D (0 past the end).
__global__ __launch_bounds__(256) void bwd_prep_kernel(float* __restrict__ Lb,
                                                       float* __restrict__ Dp,
                                                       const float* __restrict__ lse,
                                                       const float* __restrict__ D, int BH, int N,
                                                       int n_pad, int* __restrict__ ctrl, int n_ctrl,
                                                       int n_zero) {
    const long long rows = (long long)BH * n_pad;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < rows;
         i += (long long)gridDim.x * 256) {
        const long long bh = i / n_pad;
        const int n = (int)(i % n_pad);
        const bool in = n < N;
        Lb[i] = in ? lse[bh * N + n] * kLog2e : __builtin_inff();
        Dp[i] = in ? -D[bh * N + n] : 0.f;       // -D: added to dP in the kernels
    }
    // the fused kernel's control block: n_zero zeros, then "no tile yet"
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n_ctrl; i += gridDim.x * 256)
        ctrl[i] = i < n_zero ? 0 : 0x7fffffff;
}

// Grouped-query attention with the query heads of a group split over NS
// workgroups: dK = sum of the NS fp32 partials (part), dV likewise (the block
// after them), summed in part order and rounded to bf16.  n = B * Hkv * N * d
// elements of each, a multiple of 4.
__global__ __launch_bounds__(256) void gqa_reduce_kernel(const float* __restrict__ part,
                                                         __bf16* __restrict__ dK,
                                                         __bf16* __restrict__ dV, int NS, long long n) {
    for (long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4; i < 2 * n;
         i += (long long)gridDim.x * 256 * 4) {
        const bool isv = i >= n;
        const long long e = isv ? i - n : i;
        const float* src = part + (isv ? (long long)NS * n : 0) + e;
        f32x4 acc = *reinterpret_cast<const f32x4*>(src);
        for (int sp = 1; sp < NS; ++sp) acc += *reinterpret_cast<const f32x4*>(src + (long long)sp * n);
        bf16x4 out;
#pragma unroll
        for (int c = 0; c < 4; ++c) out[c] = (__bf16)acc[c];
        *reinterpret_cast<bf16x4*>((isv ? dV : dK) + e) = out;
    }
}

// ----------------------------------------------------------------------------
// Fused backward main kernel
// ----------------------------------------------------------------------------
namespace bwd {

constexpr int BC = 128;          // keys per workgroup
constexpr int BR = 64;           // query rows per iteration
constexpr int NW = 8;            // wave64s per workgroup (2 per SIMD)
constexpr int NT = NW * 64;

template <int HD> struct Smem {
    static constexpr int TILE = BR * HD * 2;              // one Q_i or dO_i tile (bytes)
    static constexpr int off_q = 0;                       // two buffers
    static constexpr int off_do = 2 * TILE;               // two buffers
    static constexpr int off_k = 4 * TILE;
    static constexpr int off_v = off_k + BC * HD * 2;
    static constexpr int off_l = off_v + BC * HD * 2;     // float[2][BR]
    static constexpr int off_d = off_l + 2 * BR * 4;      // float[2][BR]
    static constexpr int bytes = off_d + 2 * BR * 4;
    // the dK / dV partial exchange of the epilogue overlays [0, off_l)
    static constexpr int xchg = 4 * 2 * (HD / 32) * 16 * 64 * 4;
    static_assert(xchg <= off_l, "partial exchange must fit below L / D");
};

// Workspace tile of dS for one (batch*head, query tile i, 128-key tile j),
// BC x BR bf16 = 16 KiB, in the register order of its producer so that every
// store is a whole 1 KiB run: block (qh, wh) = query rows 32 qh .. + 31 and
// keys 64 wh .. + 63 is 4 KiB at (2 qh + wh) * 4 KiB; in it, 1 KiB run
// c = 2 sk + k4 holds, for lane l = kl + 32 g, the 16 bytes of key
// 64 wh + 32 sk + kl and query rows 32 qh + (2 k4 + e / 4) * 8 + 4 g + e % 4,
// e = 0..7 (the C layout of an S / dP block, rows 16 k4 .. 16 k4 + 15,
// rounded to bf16).
constexpr int DST_EL = BC * BR;

__device__ __forceinline__ int dst_run(int qh, int wh, int sk, int k4) {   // byte offset
    return (2 * qh + wh) * 4096 + (2 * sk + k4) * 1024;
}

// The dQ kernel keeps a dS tile in LDS with its 16-byte chunks permuted by
// dst_lds_chunk (an involution: bits 2..3 of the chunk index flip by bits
// 6, 5), which makes its transposing reads (4 keys x 8 query units of 4
// rows per half-wave) hit 32 distinct 8-byte bank slots.
__device__ __forceinline__ int dst_lds_chunk(int c) {
    return c ^ ((((c >> 6) & 1) << 3) | (((c >> 5) & 1) << 2));
}

// dS tiles of a (batch*head) are stored row after row of query tiles i; when
// causal only the tiles with j <= i / 2 (the lower triangle: every 128-key
// tile that reaches a row of the 64-row tile i) have a slot, i / 2 + 1 per
// row, so row i starts at sum_{i' < i} (i' / 2 + 1) = (a + 1)(a + b) for
// i = 2 a + b.
__host__ __device__ __forceinline__ long long dst_row0(int i, bool causal, int tc) {
    const long long a = i >> 1, b = i & 1;
    return causal ? (a + 1) * (a + b) : (long long)i * tc;
}

__host__ __device__ __forceinline__ long long dst_tiles_per_head(int tr, int tc, bool causal) {
    return dst_row0(tr, causal, tc);
}

__device__ __forceinline__ size_t dst_tile(int bh, int i, int j, int tr, int tc, bool causal) {
    return ((size_t)bh * dst_tiles_per_head(tr, tc, causal) + dst_row0(i, causal, tc) + j) * DST_EL;
}

// Workspace image of K_j as ready-made B operands of dQ = dS K: for each
// 32-column head-dim block db and 16-key step ks, a 1 KiB block in which lane l
// holds K[16 ks + 8 (l / 32) + e][32 db + l % 32], e = 0..7.
__device__ __forceinline__ size_t kimg_tile(int bh, int j, int tc, int HD) {
    return ((size_t)bh * tc + j) * BC * HD;
}

// ----------------------------------------------------------------------------
// Kernel A: one workgroup per (batch*head, 128-key tile j).  Walks the query
// tiles i (from the diagonal tile when causal), recomputes S_ij and P_ij from
// L, forms dP_ij and dS_ij, accumulates dV_j = sum P^T dO and dK_j = sum dS^T Q
// in registers, and stores dS_ij^T (bf16) for the dQ kernel.
//
// Eight wave64s (two per SIMD): wave (kw, qh) owns keys 32 kw .. + 31 and query
// rows 32 qh .. + 31 of each 64-row tile; the two waves that share keys add
// their dK / dV partials through LDS at the end.  Q_i / dO_i are double
// buffered in LDS by direct global -> LDS copies issued one tile ahead; K_j and
// V_j stay in LDS.  The accumulator layout of S / dP (one key per lane) is the A
// layout of P^T and dS^T, so dV and dK take P and dS straight from registers
// with the query index relabelled consistently on the B side, whose operands
// (dO, Q with one head-dim column per lane) come from transposing LDS reads.
// ----------------------------------------------------------------------------
template <int HD, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                     const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                     const float* __restrict__ Lb, const float* __restrict__ Dp,
                     __bf16* __restrict__ dSw, __bf16* __restrict__ Kimg, __bf16* __restrict__ dK,
                     __bf16* __restrict__ dV, int BH, int H, int G, int NS, float* __restrict__ part,
                     int N, int n_pad, float scale) {
    using S = Smem<HD>;
    constexpr int KSD = HD / 16;                 // k steps over the head dim
    constexpr int DB = HD / 32;                  // 32-wide blocks of the head dim
    constexpr int TILE_EL = BR * HD;             // elements of one Q_i / dO_i buffer
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int lane = threadIdx.x & 63;
    const int w = wave_id();
    const int kw = w & 3;                        // this wave's 32 keys of the 128
    const int qh = w >> 2;                       // this wave's 32 query rows of the 64
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int t16 = lane & 15;                   // lane within its 16-lane group
    const int hh = (lane >> 4) & 1;              // which 16-lane half of the 32
    const int s4 = t16 >> 2;                     // row offset inside a transposing read

    const int tc = (N + BC - 1) / BC;
    const int tr_count = (N + BR - 1) / BR;
    const int logical = xcd_remap(blockIdx.x, BH * tc);
    const int j = logical % tc;                  // heavy (small j) first when causal
    const int k0 = j * BC;
    // grouped-query attention: BH = B * (H / G) * NS workgroup rows, one per
    // (K / V head bh, part sp of its G query heads); the part's G / NS query
    // heads hq0 .. are summed in registers, the NS parts in gqa_reduce_kernel
    const int bh = (logical / tc) / NS, sp = (logical / tc) % NS;
    const int GS = G / NS;
    const size_t head = (size_t)bh * N * HD;     // K, V, dK, dV
    const int hq0 = (bh / (H / G)) * H + (bh % (H / G)) * G + sp * GS;

    __bf16* const QB = reinterpret_cast<__bf16*>(smem + S::off_q);   // Q buffers; dO at +2 tiles
    __bf16* const KB = reinterpret_cast<__bf16*>(smem + S::off_k);   // K; V at +BC*HD
    float* const LB = reinterpret_cast<float*>(smem + S::off_l);     // L buffers; D at +2*BR

    // ---- loop-invariant per-lane LDS offsets (elements, relative to a tile);
    //      every access below is one of these, XORed with a constant, plus a
    //      compile-time constant
    // row reads of the A / B operands of S and dP: chunk 2ks+g of row rq / rk;
    // k steps ks and ks + 4 differ in chunk bit 3 only (offset ^ 64)
    int oq[4], okr[4];
    {
        const int rq = qh * 32 + l32, rk = kw * 32 + l32;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            oq[i] = roff<HD>(rq, 2 * i + g);
            okr[i] = roff<HD>(rk, 2 * i + g);
        }
    }
    // transposing reads of dO_i / Q_i (B operands of dV, dK): rows
    // qh*32 + 16 k4 + 4g + s4 and those + 8, columns 32 db + 16 hh + 4 (t16 & 3).
    // The row swizzle is the same for every k4; rows + 8 flip chunk bit 1
    // (offset ^ 16) and head-dim block db flips chunk bits 2..3 by db
    // (offset ^ (db << 5)).
    const int otr = roff4<HD>(qh * 32 + g * 4 + s4, hh * 16 + 4 * (t16 & 3));
    const int ol = qh * 32 + g * 4;              // L / D rows of this lane (+ 8 rr)

    const int it0 = CAUSAL ? (k0 / BR) : 0;

    // ---- K_j, V_j and the first Q_i / dO_i tile (with its L, D rows) to LDS.
    //      Each copy's row offset lives in the buffer descriptor (scalar); the
    //      per-lane offsets are loop-invariant; rows past N read as zero.
    constexpr int ROWB = HD * 2;                 // bytes per row
    int vo_q[BR * (HD / 8) / 64 / NW], vo_k[BC * (HD / 8) / 64 / NW];
    stage_offsets<HD, BR, NW>(vo_q, w, lane);
    stage_offsets<HD, BC, NW>(vo_k, w, lane);
    auto stage_tile = [&](int gq, int it, int buf) {
        const int q0 = it * BR;
        const int bytes = min(N - q0, BR) * ROWB;
        const size_t qhd = (size_t)(hq0 + gq) * N * HD;
        const size_t qst = (size_t)(hq0 + gq) * n_pad;
        stage_rows_b<HD, BR, NW>(make_rsrc(Q + qhd + (size_t)q0 * HD, bytes), vo_q,
                                 smem + S::off_q + buf * S::TILE, w);
        stage_rows_b<HD, BR, NW>(make_rsrc(dO + qhd + (size_t)q0 * HD, bytes), vo_q,
                                 smem + S::off_do + buf * S::TILE, w);
        if (w == 0) bdma4(make_rsrc(Lb + qst + q0, BR * 4), lane * 4, smem + S::off_l + buf * BR * 4);
        if (w == 1) bdma4(make_rsrc(Dp + qst + q0, BR * 4), lane * 4, smem + S::off_d + buf * BR * 4);
    };
    {
        const int bytes = min(N - k0, BC) * ROWB;
        stage_rows_b<HD, BC, NW>(make_rsrc(K + head + (size_t)k0 * HD, bytes), vo_k, smem + S::off_k, w);
        stage_rows_b<HD, BC, NW>(make_rsrc(V + head + (size_t)k0 * HD, bytes), vo_k, smem + S::off_v, w);
    }
    const int nt = tr_count - it0;               // query tiles per query head
    stage_tile(0, it0, 0);
    __syncthreads();

    // ---- K_j image for the dQ kernel: 2 * DB * 8 blocks of 1 KiB, spread over
    //      the waves; each block is two transposing reads of the K tile
    {
        constexpr int NBLK = DB * (BC / 16);
        const __amdgpu_buffer_rsrc_t kr = make_rsrc(Kimg + kimg_tile(bh, j, tc, HD), sp == 0 ? BC * HD * 2 : 0);
#pragma unroll
        for (int b = 0; b < NBLK / NW; ++b) {
            const int blk = w * (NBLK / NW) + b;
            const int bdb = blk / (BC / 16), bks = blk % (BC / 16);
            const int key = bks * 16 + g * 8 + s4;
            const int col = bdb * 32 + hh * 16 + 4 * (t16 & 3);
            const bf16x8 v = cat44(lds_read_tr(KB + roff4<HD>(key, col)),
                                   lds_read_tr(KB + roff4<HD>(key + 4, col)));
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), kr,
                                                   (blk * 64 + lane) * 16, 0, 0);
        }
    }

    f32x16 dv[DB], dk[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) {
        dv[b] = zero16();
        dk[b] = zero16();
    }

    const float sl2 = scale * kLog2e;
    const int key_lane = k0 + kw * 32 + l32;     // this lane's key (accumulator column)

    for (int step = 0, buf = 0; step < GS * nt; ++step, buf ^= 1) {
        const int gq = step / nt, it = it0 + step % nt;
        const int q0 = it * BR;
        if (step + 1 < GS * nt)                  // lands during this iteration
            stage_tile((step + 1) / nt, it0 + (step + 1) % nt, buf ^ 1);
        const __bf16* Qs = QB + buf * TILE_EL;
        const __bf16* dOs = Qs + 2 * TILE_EL;
        const float* Ls = LB + buf * BR;
        const float* Ds = Ls + 2 * BR;

        // ---- S = Q K^T, dP = dO V^T: this wave's 32 queries x 32 keys
        f32x16 s = zero16(), dp = zero16();
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            const int xo = (ks >> 2) * 64;          // chunk bit 3 for k steps 4..7
            const int oa = oq[ks & 3] ^ xo, ob = okr[ks & 3] ^ xo;
            s = mfma32(lds_read16(Qs + oa), lds_read16(KB + ob), s);
            dp = mfma32(lds_read16(dOs + oa), lds_read16(KB + BC * HD + ob), dp);
        }

        // ---- masking, only where this wave's keys reach past its first query
        //      row (causal diagonal) or past the end (ragged last key tile)
        const bool need_mask =
            (k0 + BC > N) || (CAUSAL && (k0 + kw * 32 + 31 > q0 + qh * 32));
        if (__builtin_expect(need_mask, 0)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int q = q0 + ol + (r >> 2) * 8 + (r & 3);
                const bool masked = (key_lane >= N) || (CAUSAL && key_lane > q);
                s[r] = masked ? -__builtin_inff() : s[r];
            }
        }
        // ---- P = exp(scale*S - L), dS = P o (dP - D); masked entries give 0
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const f32x4 lv = *reinterpret_cast<const f32x4*>(Ls + ol + rr * 8);
            const f32x4 dd = *reinterpret_cast<const f32x4*>(Ds + ol + rr * 8);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = rr * 4 + e;
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, -lv[e]));
                s[r] = p;
                dp[r] = p * (dp[r] + dd[e]);      // dd holds -D
            }
        }
        // ---- P^T, dS^T as A operands (k = query, relabelled per lane group)
        const bf16x8 pa0 = pack_c8(s, 0), pa1 = pack_c8(s, 8);
        const bf16x8 ds0 = pack_c8(dp, 0), ds1 = pack_c8(dp, 8);

        // ---- dV += P^T dO, dK += dS^T Q over this wave's 32 queries; the B
        //      operands are read transposed from the row-major dO_i, Q_i tiles
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int o0 = otr ^ (db << 5);
            const int o8 = (otr + 8 * HD) ^ (db << 5) ^ 16;
#pragma unroll
            for (int k4 = 0; k4 < 2; ++k4) {
                const int rk = k4 * 16 * HD;
                const bf16x8 bo = cat44(lds_read_tr(dOs + o0 + rk), lds_read_tr(dOs + o8 + rk));
                const bf16x8 bq = cat44(lds_read_tr(Qs + o0 + rk), lds_read_tr(Qs + o8 + rk));
                dv[db] = mfma32(k4 ? pa1 : pa0, bo, dv[db]);
                dk[db] = mfma32(k4 ? ds1 : ds0, bq, dk[db]);
            }
        }
        // the next tile has landed and every read of this tile is done; the dS
        // stores go after the barrier so that its wait for the tile copies does
        // not also wait for them
        __syncthreads();
        const __amdgpu_buffer_rsrc_t dsr =
            make_rsrc(dSw + dst_tile(hq0 + gq, it, j, tr_count, tc, CAUSAL), DST_EL * 2);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, ds0), dsr,
                                               dst_run(qh, kw >> 1, kw & 1, 0) + lane * 16, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, ds1), dsr,
                                               dst_run(qh, kw >> 1, kw & 1, 1) + lane * 16, 0, 0);
    }

    // ---- epilogue: the two waves sharing 32 keys (qh = 0, 1) add their partial
    //      dK / dV through LDS; qh = 0 stores dV, qh = 1 stores dK (scaled)
    float* X = reinterpret_cast<float*>(smem);
    constexpr int PART = DB * 16 * 64;           // floats of one wave's dK (or dV)
    float* mine = X + (kw * 2 + qh) * PART;      // qh 0 publishes dK, qh 1 publishes dV
    float* other = X + (kw * 2 + (qh ^ 1)) * PART;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            mine[(db * 16 + r) * 64 + lane] = qh ? dv[db][r] : dk[db][r];
    __syncthreads();
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float tot = (qh ? dk[db][r] : dv[db][r]) + other[(db * 16 + r) * 64 + lane];
            const int key = k0 + kw * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
            if (key < N) {
                const size_t off = (size_t)key * HD + db * 32 + l32;
                if (NS > 1) {
                    // fp32 partial of part sp: dK block, then the dV block
                    const size_t bkv = BH / NS, pb = ((size_t)sp * bkv + bh) * N * HD + off;
                    if (qh) part[pb] = tot * scale;
                    else part[(size_t)NS * bkv * N * HD + pb] = tot;
                } else if (qh) {
                    dK[head + off] = (__bf16)(tot * scale);
                } else {
                    dV[head + off] = (__bf16)tot;
                }
            }
        }
    }
}

// ----------------------------------------------------------------------------
// Kernel A for d = 128, one wave per SIMD: one workgroup of 4 wave64s per
// (batch*head, 256-key tile); wave w owns keys 64 w .. + 63 (two 32-key blocks
// kb) and all 64 rows of each query tile, so every Q_i / dO_i operand read from
// LDS feeds two MFMAs (one per key block) and no dK / dV partials need
// combining.  K_j stays in VGPRs as the B operand of S = Q K^T; V_j sits in
// LDS; the dK / dV accumulators (64 keys x 128 columns each) take the
// accumulation registers.  The two 32-row halves qb of a query tile are
// processed one after the other.  dS tiles and the K image are written in
// the 128-key format the dQ kernel reads.
// ----------------------------------------------------------------------------
constexpr int BC2 = 256;                         // keys per workgroup
constexpr int NW2 = 4;

struct Smem2 {
    static constexpr int HD = 128;
    static constexpr int TILE = BR * HD * 2;              // one Q_i or dO_i buffer (16 KiB)
    static constexpr int off_q = 0;                       // two buffers
    static constexpr int off_do = 2 * TILE;               // two buffers
    static constexpr int off_v = 4 * TILE;                // V_j, 256 x 128
    static constexpr int off_l = off_v + BC2 * HD * 2;    // float[2][BR]
    static constexpr int off_d = off_l + 2 * BR * 4;      // float[2][BR]
    static constexpr int bytes = off_d + 2 * BR * 4;
    static constexpr int off_kstage = 0;                  // K_j in the prologue (overlays Q/dO)
    static_assert(BC2 * HD * 2 <= off_v, "K staging must fit below V");
};

// Causal 256-key tiles have (N - 256 j) / 64 query tiles.  Workgroups are
// dealt round-robin over the 8 XCDs (hardware index b runs on XCD b % 8);
// each XCD takes every eighth head and works through them two at a time,
// longest tiles first within each pair.  That balances the work like a
// global longest-first order while only about four heads' Q / dO are in use
// on an XCD at once (its L2 holds them).  Other head counts: all heads' tile 0
// first, then tile 1, ...  Non-causal tiles are equal; consecutive tiles of a
// head go to the same XCD.
template <bool CAUSAL>
__device__ __forceinline__ void w64_grid_item(int b, int BH, int tc2, int& bh, int& j) {
    if (CAUSAL && BH % 16 == 0) {
        const int x = b % 8, t = b / 8;
        const int grp = t / (2 * tc2), r = t % (2 * tc2);
        j = r / 2;
        bh = (2 * grp + (r & 1)) * 8 + x;
    } else if (CAUSAL) {
        bh = b % BH;
        j = b / BH;
    } else {
        const int logical = xcd_remap(b, BH * tc2);
        bh = logical / tc2;
        j = logical % tc2;
    }
}

constexpr int FQ = 4;                            // query tiles whose dQ an item forms
constexpr int F_DS_B = DST_EL * 2;               // one dS tile (bytes)
constexpr int F_CTRL = 64;                       // ints of the control block before prog
constexpr int F_WAIT_LIMIT = 1 << 22;            // polls (about 0.1 us each) before giving up

struct FusedSmem {
    static constexpr int body = Smem2::bytes;    // the dQ stages overlay the dK/dV layout
    static constexpr int ticket = body;          // the claimed ticket, broadcast to the waves
    static constexpr int state = body + 16;      // the work loop's state across an item (8 ints)
    static constexpr int bytes = body + 48;
};

// A value recomputed where it stands (an empty asm the compiler must keep in
// place): in the persistent kernel below, per-lane and per-shape constants
// derived from these would otherwise be hoisted out of its work loop and kept
// live across both phases of every item, which the register file cannot hold.
__device__ __forceinline__ int here_v(int x) {
    asm volatile("" : "+v"(x));
    return x;
}
// this lane's index in its wave, computed from nothing (threadIdx.x need not
// stay live across a persistent loop)
__device__ __forceinline__ int lane_here() {
    int x;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
    return x;
}
__device__ __forceinline__ int here_s(int x) {
    asm volatile("" : "+s"(x));
    return x;
}

// One work item of the d = 128 dK/dV kernel: key tile j (256 keys) of the
// grid row `bh` (a K / V head, times NS parts of its query heads).  FUSED:
// the item is part of the persistent causal kernel below; its dS stores stay
// cacheable (the same XCD reads them back within a few tiles) and, after
// every fourth query tile, it publishes in prog[bh * tc2 + j] the lowest
// query tile whose dS tiles are all stored.
template <bool CAUSAL, bool FUSED>
__device__ __forceinline__ void dkdv_w64_item(char* smem, const __bf16* __restrict__ Q,
                                              const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                                              const __bf16* __restrict__ dO, const float* __restrict__ Lb,
                                              const float* __restrict__ Dp, __bf16* __restrict__ dSw,
                                              __bf16* __restrict__ Kimg, __bf16* __restrict__ dK,
                                              __bf16* __restrict__ dV, int BH, int H, int G, int NS,
                                              float* __restrict__ part, int N, int n_pad, float scale,
                                              int bh, int j, int* __restrict__ prog, int wave) {
    constexpr int HD = 128;
    using S = Smem2;
    constexpr int KSD = HD / 16;                 // 8 k steps over the head dim
    constexpr int DB = HD / 32;                  // 4 column blocks
    constexpr int TILE_EL = BR * HD;

    // FUSED: the item runs inside the persistent kernel's loop, and the
    // register file is full inside the tile loop; lane, wave and N are
    // recomputed here (and the per-tile copy offsets and the mask lanes where
    // they are used) so that nothing derived from them is hoisted out of the
    // item loop and held across it, which would spill inside the tile loop
    const int lane = FUSED ? lane_here() : (int)(threadIdx.x & 63);
    const int w = FUSED ? here_s(wave) : wave_id();
    if (FUSED) N = here_s(N);
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int t16 = lane & 15;
    const int hh = (lane >> 4) & 1;
    const int s4 = t16 >> 2;

    const int tc = (N + BC - 1) / BC;            // 128-key tiles (dS and K image format)
    const int tr_count = (N + BR - 1) / BR;
    const int k0 = j * BC2;
    const int kw0 = k0 + 64 * w;                 // this wave's first key

    // grouped-query attention: the mapped row is (K / V head, part sp of its
    // G query heads); the part's G / NS query heads hq0 .. are summed in
    // registers, the NS parts in gqa_reduce_kernel
    const int sp = bh % NS;
    bh /= NS;
    const int GS = G / NS;
    const size_t head = (size_t)bh * N * HD;     // K, V, dK, dV
    const int hq0 = (bh / (H / G)) * H + (bh % (H / G)) * G + sp * GS;
    const __bf16* VS = reinterpret_cast<const __bf16*>(smem + S::off_v);
    const __bf16* KS = reinterpret_cast<const __bf16*>(smem + S::off_kstage);

    // row reads: chunk 2 i + g of row l32 (+ a multiple of 16 rows keeps the
    // swizzle); k steps 4..7 flip chunk bit 3 (offset ^ 64)
    // (2 ks + g) ^ swz = ((g ^ swz) & 1 | (swz & ~1) ^ 2 ks): offset ob0 ^ 16 ks
    const int ob0 = roff<HD>(l32, g);
    // transposing reads of dO_i / Q_i: rows 4 g + s4 (+ 16 k4, + 32 qb, + 8),
    // columns 16 hh + 4 (t16 & 3) (+ 32 db)
    const int otr = roff4<HD>(g * 4 + s4, hh * 16 + 4 * (t16 & 3));
    const int it0 = CAUSAL ? (k0 / BR) : 0;

    // ---- K_j, V_j into LDS; then K_j into registers and the K image
    constexpr int ROWB = HD * 2;
    int vo_k[BC2 * (HD / 8) / 64 / NW2];
    stage_offsets<HD, BC2, NW2>(vo_k, w, lane);
    {
        const int rows = min(N - k0, BC2);
        stage_rows_b<HD, BC2, NW2>(make_rsrc(K + head + (size_t)k0 * HD, rows * ROWB), vo_k,
                                   smem + S::off_kstage, w);
        stage_rows_b<HD, BC2, NW2>(make_rsrc(V + head + (size_t)k0 * HD, rows * ROWB), vo_k,
                                   smem + S::off_v, w);
    }
    __syncthreads();
    bf16x8 kreg[2][KSD];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks)
            kreg[kb][ks] = lds_read16(KS + (ob0 ^ (ks * 16)) + (64 * w + 32 * kb) * HD);
    {
        // 128-key image tile jt = w >> 1 of this workgroup; 32 blocks of 1 KiB,
        // 16 per wave.  One image per K / V head, written by part 0; FUSED:
        // one per query head (hq0, the item's only query head), which the
        // dQ phases of that head's later items read
        const int jt = w >> 1, jg = 2 * j + jt;
        if (jg < tc && (FUSED || sp == 0)) {
            const __amdgpu_buffer_rsrc_t kr =
                make_rsrc(Kimg + kimg_tile(FUSED ? hq0 : bh, jg, tc, HD), BC * HD * 2);
#pragma unroll
            for (int b = 0; b < 16; ++b) {
                const int blk = (w & 1) * 16 + b;
                const int bdb = blk / (BC / 16), bks = blk % (BC / 16);
                const int key = jt * BC + bks * 16 + g * 8 + s4;
                const int col = bdb * 32 + hh * 16 + 4 * (t16 & 3);
                const bf16x8 v = cat44(lds_read_tr(KS + roff4<HD>(key, col)),
                                       lds_read_tr(KS + roff4<HD>(key + 4, col)));
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), kr,
                                                       (blk * 64 + lane) * 16, 0, 0);
            }
        }
    }
    __syncthreads();                             // K staging consumed

    auto stage_tile = [&](int gq, int it, int buf) {
        const int q0 = it * BR;
        const int bytes = min(N - q0, BR) * ROWB;
        const size_t qhd = (size_t)(hq0 + gq) * N * HD;
        const size_t qst = (size_t)(hq0 + gq) * n_pad;
        int vo_q[BR * (HD / 8) / 64 / NW2];
        stage_offsets<HD, BR, NW2>(vo_q, FUSED ? here_s(w) : w, FUSED ? lane_here() : lane);
        stage_rows_b<HD, BR, NW2>(make_rsrc(Q + qhd + (size_t)q0 * HD, bytes), vo_q,
                                  smem + S::off_q + buf * S::TILE, w);
        stage_rows_b<HD, BR, NW2>(make_rsrc(dO + qhd + (size_t)q0 * HD, bytes), vo_q,
                                  smem + S::off_do + buf * S::TILE, w);
        if (w == 0) bdma4(make_rsrc(Lb + qst + q0, BR * 4), lane * 4, smem + S::off_l + buf * BR * 4);
        if (w == 1) bdma4(make_rsrc(Dp + qst + q0, BR * 4), lane * 4, smem + S::off_d + buf * BR * 4);
    };
    // query tiles are walked from the last one down to the diagonal: the
    // workgroups of one head then read the same Q_i / dO_i at the same time,
    // and the shared L2 serves all but the first
    const int nt = tr_count - it0;               // query tiles per query head
    stage_tile(0, tr_count - 1, 0);
    __syncthreads();

    f32x16 dv[2][DB], dk[2][DB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int b = 0; b < DB; ++b) {
            dv[kb][b] = zero16();
            dk[kb][b] = zero16();
        }
    const float sl2 = scale * kLog2e;
    // dS stores: keys (w & 1) * 64 .. + 63 of 128-key tile 2 j + (w >> 1)
    const int jst = 2 * j + (w >> 1);
    // row reads of V_j: this wave's rows, k step ks at ^ 32 ks bytes, key
    // block 1 at + 8 KiB
    const uint32_t aV = lds_addr(VS) + (uint32_t)((64 * w * HD + ob0) * 2);
    uint32_t aVx[KSD];
    static_for<0, KSD>([&](auto ksI) {
        constexpr int ks = decltype(ksI)::value;
        aVx[ks] = vxor<ks * 32>(aV);
    });

    for (int step = 0, buf = 0; step < GS * nt; ++step, buf ^= 1) {
        const int gq = step / nt, it = tr_count - 1 - step % nt;
        const int q0 = it * BR;
        if (step + 1 < GS * nt)                  // lands during this iteration
            stage_tile((step + 1) / nt, tr_count - 1 - (step + 1) % nt, buf ^ 1);
        const __bf16* Qs = reinterpret_cast<const __bf16*>(smem + S::off_q) + buf * TILE_EL;
        const float* Ls = reinterpret_cast<const float*>(smem + S::off_l) + buf * BR;
        // dS stores go nowhere (buffer records 0) for a 128-key half past N,
        // or above the diagonal when causal (no slot: every entry is masked)
        const bool st_ok = jst < tc && (!CAUSAL || jst <= it / 2);
        const __amdgpu_buffer_rsrc_t dsr =
            make_rsrc(dSw + dst_tile(hq0 + gq, it, st_ok ? jst : 0, tr_count, tc, CAUSAL), st_ok ? DST_EL * 2 : 0);
        // transposing-read bases of this tile: Q buffer + lane offset for the
        // 4 column blocks x 2 row halves; dO, the row half qb and k4 are
        // immediate offsets
        uint32_t trv[DB][2];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            trv[db][0] = lds_addr(Qs) + (uint32_t)((otr ^ (db << 5)) * 2);
            trv[db][1] = lds_addr(Qs) + (uint32_t)((((otr + 8 * HD) ^ (db << 5)) ^ 16) * 2);
        }
        // row-read bases of this tile: Q rows of this lane (k step ks at
        // ^ 32 ks bytes; dO at + 32 KiB, row half 1 at + 8 KiB) and L (D at
        // + 512 bytes)
        const uint32_t aQ = lds_addr(Qs) + (uint32_t)(ob0 * 2);
        const uint32_t aL = lds_addr(Ls) + (uint32_t)(g * 16);
        // the k-step addresses of the row reads, once per tile (the swizzle
        // is an XOR, which no immediate offset can express)
        uint32_t aQx[KSD];
        static_for<0, KSD>([&](auto ksI) {
            constexpr int ks = decltype(ksI)::value;
            aQx[ks] = vxor<ks * 32>(aQ);
        });

        // L of row group 0 of half h, its Q operands for S and its -D (the
        // initial value of the dP accumulators), loaded ahead
        f32x4 lv[4], dd[4];
        bf16x8 aq[KSD];
        auto load_s = [&](auto hI) {
            constexpr int h = decltype(hI)::value;
            lds_ld<h * 128>(lv[0], aL);
            static_for<0, KSD>([&](auto ksI) {
                constexpr int ks = decltype(ksI)::value;
                lds_ld<h * 8192>(aq[ks], aQx[ks]);
            });
            static_for<0, 4>([&](auto rrI) {
                constexpr int rr = decltype(rrI)::value;
                lds_ld<512 + h * 128 + rr * 32>(dd[rr], aL);
            });
        };
        load_s(std::integral_constant<int, 0>{});
        static_for<0, 2>([&](auto qbI) {
            constexpr int qb = decltype(qbI)::value;
            using SC = W64Sched;
            // A half runs four phases of 16 MFMAs: S, dP, dV, dK.  The
            // softmax VALU work is spread over the dP phase (P and its bf16
            // packing) and the dV phase (dS = P o (dP - D) and its packing;
            // the dP accumulators start from -D, so that is one product),
            // one share after each MFMA, so that it issues while the matrix
            // core works on the previous product; each slot ends in a
            // sched_barrier that keeps the compiler from regrouping it.
            // Elements are taken in the order (row group rr, key block kb).
            // Every LDS read is issued from assembly at a fixed point of
            // this schedule and waited for with the count W64Sched derives.
            bf16x8 ado[KSD], bv[KSD][2];
            auto load_dp = [&](auto ksI) {
                constexpr int ks = decltype(ksI)::value;
                lds_ld<2 * S::TILE + qb * 8192>(ado[ks], aQx[ks]);
                lds_ld<0>(bv[ks][0], aVx[ks]);
                lds_ld<8192>(bv[ks][1], aVx[ks]);
            };
            // step t = 4 k4 + db of the dV (src dO) or dK (src Q) phase
            u32x2 tb[8][2];
            auto tr_step = [&](auto tI, auto doI) {
                constexpr int t = decltype(tI)::value, db = t & 3, k4 = t >> 2;
                constexpr int off = (qb * 32 * HD + k4 * 16 * HD) * 2 + (decltype(doI)::value ? 2 * S::TILE : 0);
                tr_read2o<off>(tb[t][0], tb[t][1], trv[db][0], trv[db][1]);
            };
            using IsDo = std::integral_constant<int, 1>;
            using IsQ = std::integral_constant<int, 0>;
            f32x16 s[2], dp[2];
            // ---- S = Q K^T: 32 queries x 64 keys
            static_for<0, KSD>([&](auto ksI) {
                constexpr int ks = decltype(ksI)::value;
                lgkm_wait<SC::wait_S(ks)>(aq[ks]);
                static_for<0, 2>([&](auto kbI) {
                    constexpr int kb = decltype(kbI)::value;
                    if constexpr (ks == 0) mfma_v0(s[kb], aq[ks], kreg[kb][ks]);
                    else mfma_v(s[kb], aq[ks], kreg[kb][ks]);
                });
                if constexpr (SC::S_LD(ks) > 0) load_dp(std::integral_constant<int, ks - (KSD - SC::PD)>{});
                __builtin_amdgcn_sched_barrier(0);
            });
            mfma_v_settle2(s[0], s[1]);
            __builtin_amdgcn_sched_barrier(0);
            // ---- masking where this block's keys reach past its first query
            //      row (causal diagonal) or past the end
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int kb0 = kw0 + 32 * kb;
                const bool need_mask = (kb0 + 32 > N) || (CAUSAL && (kb0 + 31 > q0 + 32 * qb));
                if (__builtin_expect(need_mask, 0)) {
                    const int lm = FUSED ? lane_here() : lane;
                    const int key = kb0 + (lm & 31);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int q = q0 + 32 * qb + (r >> 2) * 8 + (lm >> 5) * 4 + (r & 3);
                        const bool masked = (key >= N) || (CAUSAL && key > q);
                        s[kb][r] = masked ? -__builtin_inff() : s[kb][r];
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            // ---- dP = dO V^T; VALU slots: P = 2^(S scale log2 e - L log2 e)
            bf16x8 pa[2][2], da[2][2];
            static_for<0, 16>([&](auto mI) {
                constexpr int m = decltype(mI)::value, ks = m >> 1, kb = m & 1, rr = m >> 2;
                if constexpr (m == 12) tr_step(std::integral_constant<int, 0>{}, IsDo{});
                if constexpr (m == 14) tr_step(std::integral_constant<int, 1>{}, IsDo{});
                if constexpr (SC::P_DP(m) > 0) load_dp(std::integral_constant<int, ks + SC::PD>{});
                if constexpr (SC::P_LV(m) > 0) lds_ld<qb * 128 + (rr + 1) * 32>(lv[rr + 1], aL);
                // each register is tied to the first wait that covers it only
                // (-D came with the half's first reads, before dO step 0)
                if constexpr (m == 0)
                    asm volatile("s_waitcnt lgkmcnt(%[n])"
                                 : "+v"(ado[0]), "+v"(bv[0][0]), "+v"(lv[0]), "+v"(dd[0]), "+v"(dd[1]),
                                   "+v"(dd[2]), "+v"(dd[3])
                                 : [n] "n"(SC::wait_P(0) > 15 ? 15 : SC::wait_P(0)));
                else if constexpr (kb == 1)
                    lgkm_wait<SC::wait_P(m)>(bv[ks][1]);
                else if constexpr ((m & 3) == 0)
                    lgkm_wait<SC::wait_P(m)>(ado[ks], bv[ks][0], lv[rr]);
                else
                    lgkm_wait<SC::wait_P(m)>(ado[ks], bv[ks][0]);
                if constexpr (ks == 0) {
                    // dP starts from -D: row m of the C layout holds D of
                    // query row 8 (r / 4) + 4 g + r % 4, which dd[r / 4]
                    // holds in its element r % 4
                    f32x16 dinit;
#pragma unroll
                    for (int r = 0; r < 16; ++r) dinit[r] = dd[r >> 2][r & 3];
                    mfma_vc(dp[kb], ado[0], bv[0][kb], dinit);
                } else {
                    mfma_v(dp[kb], ado[ks], bv[ks][kb]);
                }
                constexpr int ekb = (m >> 1) & 1;
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int r = 4 * rr + 2 * (m & 1) + x;
                    s[ekb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[ekb][r], sl2, -lv[rr][r & 3]));
                }
                if constexpr (m == 8 || m == 9) pa[m - 8][0] = pack_c8(s[m - 8], 0);
                __builtin_amdgcn_sched_barrier(0);
            });
            mfma_v_settle2(dp[0], dp[1]);
            __builtin_amdgcn_sched_barrier(0);
            // ---- dV += P^T dO; VALU slots: dS = P o (dP - D)
            static_for<0, 16>([&](auto mI) {
                constexpr int m = decltype(mI)::value, t = m >> 1, kb = m & 1, rr = m >> 2;
                if constexpr (kb == 0) {
                    // two steps of reads stay in flight: this phase's, then
                    // the first two of the dK phase
                    if constexpr (t + 2 < 8) tr_step(std::integral_constant<int, t + 2>{}, IsDo{});
                    else tr_step(std::integral_constant<int, t - 6>{}, IsQ{});
                }
                if constexpr (kb == 0) lgkm_wait<SC::wait_V(m)>(tb[t][0], tb[t][1]);
                if constexpr (m == 0 || m == 1) pa[m][1] = pack_c8(s[m], 8);
                mfma_a(dv[kb][t & 3], pa[kb][t >> 2], cat_u(tb[t][0], tb[t][1]));
                constexpr int ekb = (m >> 1) & 1;
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int r = 4 * rr + 2 * (m & 1) + x;
                    dp[ekb][r] = s[ekb][r] * dp[ekb][r];     // dP already holds dP - D
                }
                if constexpr (m == 8 || m == 9) da[m - 8][0] = pack_c8(dp[m - 8], 0);
                __builtin_amdgcn_sched_barrier(0);
            });
            // ---- dK += dS^T Q; dS stores for the dQ kernel
            static_for<0, 16>([&](auto mI) {
                constexpr int m = decltype(mI)::value, t = m >> 1, kb = m & 1;
                if constexpr (SC::K_LD(m) > 0) tr_step(std::integral_constant<int, t + 2>{}, IsQ{});
                if constexpr (kb == 0) lgkm_wait<SC::wait_K(m)>(tb[t][0], tb[t][1]);
                if constexpr (m == 0 || m == 1) da[m][1] = pack_c8(dp[m], 8);
                if constexpr (m >= 2 && m < 6) {
                    // run (sk, k4) = (0, 0) (1, 0) (0, 1) (1, 1) of this wave's block
                    constexpr int sk = m & 1, k4 = (m - 2) >> 1;
                    // non-temporal when a second kernel reads dS much
                    // later: the tiles should not push the shared Q / dO
                    // out of L2.  FUSED: device scope (sc1), written through
                    // to memory at once while the line stays in L2 for the
                    // reads that come soon; the later ones find it in memory
                    // and its eviction costs nothing (0.5% faster than a
                    // plain write-back store, 3% faster than non-temporal).
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, da[sk][k4]), dsr,
                                                           dst_run(qb, w & 1, sk, k4) + lane * 16, 0,
                                                           FUSED ? 16 : 2);
                }
                mfma_a(dk[kb][t & 3], da[kb][t >> 2], cat_u(tb[t][0], tb[t][1]));
                // the next half's L and Q operands, after the last wait
                if constexpr (qb == 0 && m == 15) load_s(std::integral_constant<int, 1>{});
                __builtin_amdgcn_sched_barrier(0);
            });
        });
        if constexpr (FUSED) {
            // every wave's dS stores of this tile have completed (in the
            // L2 this XCD shares) before the barrier
            if (it % 4 == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        __syncthreads();                         // next tile landed; this one free
        if constexpr (FUSED) {
            if (it % 4 == 0 && w == 0 && lane == 0) {
                // the progress slot's address waits in LDS (no register
                // holds it across the loop)
                const int* st = reinterpret_cast<const int*>(smem + FusedSmem::state);
                int* slot = reinterpret_cast<int*>(((uint64_t)(uint32_t)st[5] << 32) | (uint32_t)st[4]);
                __hip_atomic_store(slot, it, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }

    // ---- epilogue: dV, dK (scaled) of this wave's 64 keys, each pair of
    //      tiles once its last accumulations have left the matrix core.  One
    //      settle per pair: a single settle over all sixteen makes the
    //      compiler regroup the registers first, and its moves would read
    //      the last product's tile before that product has landed.
    //      Element r of tile (kb, db) is key 32 kb + 8 (r / 4) + 4 g + r % 4
    //      of the wave, column 32 db + l32.
    if (NS > 1) {
        // fp32 partials of part sp (the dK block, then the dV block) through
        // buffer resources over this wave's valid keys, laid out as the bf16
        // stores below
        const size_t bkv = BH / NS, pb0 = ((size_t)sp * bkv + bh) * N * HD;
        const size_t pv = (size_t)NS * bkv * N * HD;
        const int kwu = __builtin_amdgcn_readfirstlane(kw0);
        const int nkb = __builtin_amdgcn_readfirstlane(max(0, min(64, N - kwu)) * HD * 4);
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(part + pb0 + (size_t)kwu * HD, nkb);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(part + pv + pb0 + (size_t)kwu * HD, nkb);
        const int le = FUSED ? lane_here() : lane;
        const int vo = (4 * (le >> 5) * HD + (le & 31)) * 4;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                asm volatile("s_nop 15\n\ts_nop 7" : "+a"(dv[kb][db]), "+a"(dk[kb][db]));
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int so = (32 * kb + 8 * (r >> 2)) * HD * 4;
                    const int io = ((r & 3) * HD + db * 32) * 4;
                    // the dV element is moved to a vector register first: a
                    // store straight from the accumulation register file came
                    // out with one source register for all sixteen elements
                    float x = dv[kb][db][r];
                    asm volatile("" : "+v"(x));
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, dk[kb][db][r] * scale), rk,
                                                          vo + io, so, 0);
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, x), rv, vo + io, so, 0);
                }
            }
    } else {
        // bf16 through buffer resources over this wave's valid keys (keys at
        // or past N fall outside them and are dropped): a lane offset, the
        // key block 32 kb + 8 (r / 4) as the scalar offset, the rest immediate
        // (readfirstlane: the values are wave-uniform, and a resource the
        // compiler keeps in VGPRs turns every store into a waterfall loop)
        const int kwu = __builtin_amdgcn_readfirstlane(kw0);
        const int nkb = __builtin_amdgcn_readfirstlane(max(0, min(64, N - kwu)) * HD * 2);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(dV + head + (size_t)kwu * HD, nkb);
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(dK + head + (size_t)kwu * HD, nkb);
        // FUSED: the lane recomputed here rather than kept live over the loop
        const int le = FUSED ? lane_here() : lane;
        const int vo = (4 * (le >> 5) * HD + (le & 31)) * 2;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                asm volatile("s_nop 15\n\ts_nop 7" : "+a"(dv[kb][db]), "+a"(dk[kb][db]));
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int so = (32 * kb + 8 * (r >> 2)) * HD * 2;
                    const int io = ((r & 3) * HD + db * 32) * 2;
                    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(short, (__bf16)dv[kb][db][r]), rv,
                                                          vo + io, so, 0);
                    __builtin_amdgcn_raw_buffer_store_b16(
                        __builtin_bit_cast(short, (__bf16)(dk[kb][db][r] * scale)), rk, vo + io, so, 0);
                }
            }
    }
}

template <bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(NW2 * 64, NW2 * 64), amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_w64_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                         const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                         const float* __restrict__ Lb, const float* __restrict__ Dp,
                         __bf16* __restrict__ dSw, __bf16* __restrict__ Kimg,
                         __bf16* __restrict__ dK, __bf16* __restrict__ dV, int BH, int H, int G, int NS,
                         float* __restrict__ part, int N, int n_pad, float scale) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    int bh, j;
    w64_grid_item<CAUSAL>(blockIdx.x, BH, (N + BC2 - 1) / BC2, bh, j);
    dkdv_w64_item<CAUSAL, false>(smem, Q, K, V, dO, Lb, Dp, dSw, Kimg, dK, dV, BH, H, G, NS, part, N,
                                 n_pad, scale, bh, j, nullptr, 0);
}

// ----------------------------------------------------------------------------
// Kernel B: dQ_i = scale * sum_j dS_ij K_j, one workgroup of 4 wave64s per
// (batch*head, pair of 64-row query tiles i0 = 2 p, i1 = 2 p + 1), so that
// every K image tile loaded serves 128 query rows (both tiles of a pair see
// the same key tiles, also when causal).  Wave w owns head-dim columns
// 32 (w % DB) .. + 31 and TQ = 4 DB / 4 blocks of 32 rows.  Per key step the
// two dS tiles are copied into one of two LDS stages (the next step's copy
// runs during this step's products) and read transposed (A operands); the
// wave's K image slice comes into registers, also one step ahead.  Two
// workgroups share a CU.  The reduction over key tiles happens in fp32
// registers (no atomics).
// ----------------------------------------------------------------------------
constexpr int QW = 4;                            // waves per dQ workgroup

template <int HD, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(QW * 64, QW * 64)))
void bwd_dq_kernel(const __bf16* __restrict__ Kimg, const __bf16* __restrict__ dSw,
                   __bf16* __restrict__ dQ, int BH, int H, int G, int N, float scale) {
    constexpr int DB = HD / 32;
    constexpr int TQ = 4 * DB / QW;              // 32-row query blocks per wave (4 or 2)
    constexpr int DS_B = DST_EL * 2;             // one dS tile (bytes)
    constexpr int STB = 2 * DS_B;                // one stage: the pair's two tiles
    constexpr int NST = 2;
    constexpr int KS = BC / 16;                  // k steps per key tile
    __shared__ __attribute__((aligned(16))) char smem[NST * STB];

    const int lane = threadIdx.x & 63;
    const int w = wave_id();
    const int db = w % DB;                       // this wave's 32 head-dim columns
    const int qb0 = (w / DB) * TQ;               // its first 32-row block of the pair
    const int g = lane >> 5;
    const int t16 = lane & 15;
    const int hh = (lane >> 4) & 1;
    const int s4 = t16 >> 2;

    const int tc = (N + BC - 1) / BC;
    const int tr_count = (N + BR - 1) / BR;
    const int tp = (tr_count + 1) / 2;
    const int logical = xcd_remap(blockIdx.x, BH * tp);
    const int bh = logical / tp;
    // causal: the last pairs see the most key tiles, so they go first
    const int pr = CAUSAL ? (tp - 1 - logical % tp) : (logical % tp);
    const int i0 = 2 * pr;
    const bool has_i1 = i0 + 1 < tr_count;
    const int q0 = i0 * BR;
    const int j_end = CAUSAL ? min(tc, (min(q0 + 2 * BR, N) - 1) / BC + 1) : tc;

    // transposing reads of the A operand (dS, query rows x keys): for block
    // qb = qb0 + t (tile qb / 2, its block qb % 2) the lanes of a 16-lane
    // group address keys 16 ks + 8 g + s4 (+ 4) and the 8-byte half
    // (t16 >> 1) & 1 of query unit 4 hh + (t16 & 3); the stage and the k step
    // (keys 16 ks: chunk + 16 (ks & 1) + 128 ((ks >> 1) & 1) + 256 (ks >> 2))
    // are immediate offsets
    uint32_t tra[TQ][2];
#pragma unroll
    for (int t = 0; t < TQ; ++t)
#pragma unroll
        for (int h4 = 0; h4 < 2; ++h4) {
            const int qb = qb0 + t;
            const int c = (qb & 1) * 512 + hh * 64 + 32 * (t16 & 1) + g * 8 + h4 * 4 + s4;
            tra[t][h4] = lds_addr(smem) + (uint32_t)((qb >> 1) * DS_B + dst_lds_chunk(c) * 16 + ((t16 >> 1) & 1) * 8);
        }

    // the pair's two dS tiles of key tile jj into stage st (the second reads
    // as zero when the pair has one tile)
    auto stage = [&](int jj, int st) {
#pragma unroll
        for (int k = 0; k < STB / 1024 / QW; ++k) {
            const int I = w * (STB / 1024 / QW) + k;           // 1 KiB block of the stage
            const int t2 = I / (DS_B / 1024);
            const int Ib = I % (DS_B / 1024);
            const bool ok = t2 == 0 || has_i1;
            const __amdgpu_buffer_rsrc_t r =
                make_rsrc(dSw + dst_tile(bh, ok ? i0 + t2 : i0, jj, tr_count, tc, CAUSAL), ok ? DS_B : 0);
            bdma16_nt(r, dst_lds_chunk(Ib * 64 + lane) * 16, smem + st * STB + I * 1024);
        }
    };
    // K image loads from assembly: the compiler cannot follow which register
    // set a load in flight belongs to and would wait for the newest ones; the
    // step's own vmcnt wait covers them
    const uint32_t kvo = (uint32_t)((db * KS * 64 + lane) * 16);
    auto load_k = [&](int jj, bf16x8* kb) {
        const __bf16* kt = Kimg + kimg_tile(kv_head(bh, H, G), jj, tc, HD);
        static_for<0, KS>([&](auto ksI) {
            constexpr int ks = decltype(ksI)::value;
            gload16<(ks & 3) * 1024>(kb[ks], kt, kvo + (ks >> 2) * 4096);
        });
    };

    // Steps run one ahead: step jj's tiles sit in LDS stage jj % 2 and its K
    // slice in kb[jj % 2].  Every step, including a padding step that rounds
    // the loop up to an even count (it computes nothing), issues the loads of
    // step jj + 1 (the last real step when past the end), so at the start of
    // step jj exactly its own loads are in flight.  No load is conditional: a
    // register set written on one path only would make the compiler copy it
    // while its load may still be in flight.
    bf16x8 kb[NST][KS];
    f32x16 acc[TQ];
#pragma unroll
    for (int t = 0; t < TQ; ++t) acc[t] = zero16();
    stage(0, 0);
    load_k(0, kb[0]);
    auto step = [&](int jj, auto stI) {
        constexpr int st = decltype(stI)::value;
        vm_wait<0>(kb[st]);
        __builtin_amdgcn_s_barrier();           // step jj landed for every wave; the other stage is free
        stage(min(jj + 1, j_end - 1), st ^ 1);
        load_k(min(jj + 1, j_end - 1), kb[st ^ 1]);
        if (jj >= j_end) return;
        // A operands: transposing reads issued from assembly two k steps
        // ahead (the compiler would wait for every tile copy in flight
        // before its own), 2 TQ reads per k step
        u32x2 ta[KS][TQ][2];
        auto issue = [&](auto ksI) {
            constexpr int ks = decltype(ksI)::value;
            constexpr int off = st * STB + 256 * (ks & 1) + 2048 * ((ks >> 1) & 1) + 4096 * (ks >> 2);
#pragma unroll
            for (int t = 0; t < TQ; ++t) tr_read2o<off>(ta[ks][t][0], ta[ks][t][1], tra[t][0], tra[t][1]);
        };
        issue(std::integral_constant<int, 0>{});
        issue(std::integral_constant<int, 1>{});
        static_for<0, KS>([&](auto ksI) {
            constexpr int ks = decltype(ksI)::value;
            if constexpr (ks + 2 < KS) issue(std::integral_constant<int, ks + 2>{});
            constexpr int later = (ks + 2 < KS ? 2 : KS - 1 - ks) * 2 * TQ;
            static_for<0, TQ>([&](auto tI) {
                constexpr int t = decltype(tI)::value;
                lgkm_wait<later + 2 * (TQ - 1 - t)>(ta[ks][t][0], ta[ks][t][1]);
                acc[t] = mfma32(cat_u(ta[ks][t][0], ta[ks][t][1]), kb[st][ks], acc[t]);
            });
        });
    };
    for (int jj = 0; jj < j_end; jj += NST) {
        step(jj, std::integral_constant<int, 0>{});
        step(jj + 1, std::integral_constant<int, 1>{});
    }
    vm_wait<0>(kb[0]);                           // no copy into LDS outlives the workgroup

    // ---- dQ = scale * acc, bf16 (RNE), through a buffer resource over the
    //      pair's rows (rows past the end fall outside it and are dropped):
    //      element r of block t is row 32 (qb0 + t) + 8 (r / 4) + 4 g + r % 4
    //      of the pair, column 32 db + l32
    const int l32 = lane & 31;
    const int q0u = __builtin_amdgcn_readfirstlane(q0);
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(dQ + (size_t)bh * N * HD + (size_t)q0u * HD,
                  __builtin_amdgcn_readfirstlane(max(0, min(2 * BR, N - q0u)) * HD * 2));
    const int vo = (4 * g * HD + db * 32 + l32) * 2;
#pragma unroll
    for (int t = 0; t < TQ; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int so = ((qb0 + t) * 32 + 8 * (r >> 2)) * HD * 2;
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(short, (__bf16)(acc[t][r] * scale)), rq,
                                                  vo + (r & 3) * HD * 2, so, 0);
        }
    }
}

// ----------------------------------------------------------------------------
// Fused causal backward for d = 128 with one query head per K / V head: one
// persistent kernel in which each work item is a 256-key tile j of a head.
// The item runs the dK/dV loop above (which stores every dS tile of its keys),
// then forms dQ for the four 64-row query tiles 4 j .. 4 j + 3 of the same
// head: dQ_i = scale * sum over 128-key tiles jt <= i / 2 of dS_{i,jt} K_jt.
// Those dS tiles come from the items j' <= j of the head, which walk the
// query tiles from the last one down and so pass tiles 4 j .. 4 j + 3 one
// step before item j finishes its own loop: the tiles are read back from the
// cache while it still holds them, instead of by a second kernel after the
// whole 2 GB at the headline shape has gone to memory and back.
//
// Work queues: head bh belongs to queue bh % 8, and a workgroup takes items
// only from the queue of the XCD it runs on (hardware register XCC_ID), so
// every item of a head, and every read of what its items wrote, stays within
// one XCD and its L2.  Items are claimed with an atomic ticket in a fixed
// order: heads two at a time, key tiles heaviest (j = 0) first, the two heads'
// tiles alternating.  Item j waits only for items j' < j of its head, which
// come earlier in the same queue and were therefore claimed by workgroups
// that are running or done: no item waits for one that has not started.
// The wait is bounded; on the bound it sets a flag in the control block and
// goes on.  Tickets that no workgroup of their XCD took are processed by a
// one-workgroup sweep kernel launched right after.
//
// Control block (ints at the start of the workspace, cleared by the prep
// kernel): [0, 8) the queue tickets, [8] workgroups finished, [9] nonzero if
// a wait reached its bound, [10] items taken by the sweep kernel; then
// prog[bh * tc2 + j], the lowest query tile whose dS item j has stored (a
// multiple of 4; INT_MAX before its first).
// ----------------------------------------------------------------------------
__device__ __forceinline__ int xcc_id() {
    unsigned x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    return (int)(x & 7);
}

// Buffer -> LDS copy of dS that misses the CU's L1 (sc0: the data was written
// by other CUs of this XCD during this kernel) and is non-temporal (nt): each
// dS tile is read exactly once, and streaming it keeps the caches for the
// Q / dO tiles and K images that several items share (2.8% faster at the
// causal B8 H16 N4096 d128 shape than with sc0 alone, same results).
__device__ __forceinline__ void bdma16_l2(__amdgpu_buffer_rsrc_t r, int voff, void* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16,
                                             voff, 0, 0, 3);
}

// s_waitcnt vmcnt(N) tied to the four registers (one 64-key step of K image
// operands) whose loads it completes
template <int N>
__device__ __forceinline__ void vm_wait4(bf16x8* r) {
    static_assert(N >= 0 && N < 64, "vmcnt");
    asm volatile("s_waitcnt vmcnt(%[n])" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]) : [n] "n"(N) : "memory");
}

// dQ of the query tiles i0 .. i0 + FQ - 1 (rows past N dropped) of head bh,
// from its dS tiles and K image, in steps of 64 keys (half a 128-key dS
// tile).  Wave w owns head-dim columns 32 w .. + 31 and all 8 blocks of 32
// rows.  Each step copies the 64-key halves of the FQ dS tiles into one of
// F_NST LDS stages (wave w copies tile i0 + w) and loads the wave's K image
// slice into registers; the copies run F_NST - 1 steps ahead, so three
// steps of dS and K are in flight while one is multiplied.  The A operands
// (dS, query rows x keys) come from transposing LDS reads.
constexpr int F_HB = F_DS_B / 2;                 // one 64-key half of a dS tile (8 KiB)
constexpr int F_NST = 4;                         // dQ stages
constexpr int F_STH = FQ * F_HB;                 // one stage: the halves of the FQ tiles (32 KiB)
constexpr int F_STEP_VM = F_HB / 1024 + 4;       // vector-memory loads one step issues per wave
static_assert(F_NST * F_STH <= Smem2::bytes, "dQ stages overlay the dK/dV layout");

__device__ __forceinline__ void fused_dq_phase(char* smem, const __bf16* __restrict__ Kimg,
                                               const __bf16* __restrict__ dSw, __bf16* __restrict__ dQ,
                                               int bh, int i0, int N, float scale, int wave) {
    constexpr int HD = 128;
    constexpr int TQ = 2 * FQ;                   // 32-row blocks
    constexpr int KH = BC / 32;                  // k steps per 64-key half
    // lane and wave recomputed here: shared with the dK/dV phase, their
    // derived offsets would stay live across it
    const int lane = lane_here();
    const int w = here_s(wave);
    const int db = w;
    const int g = lane >> 5;
    const int t16 = lane & 15;
    const int hh = (lane >> 4) & 1;
    const int s4 = t16 >> 2;
    const int tc = (N + BC - 1) / BC;
    const int tr_count = (N + BR - 1) / BR;
    const int q_end = min(N, (i0 + FQ) * BR);    // one past the last row
    const int nh = 2 * min(tc, (q_end - 1) / BC + 1);   // 64-key steps

    // Layout of a stage: tile t of the FQ at t * F_HB; in it, the 4 KiB block
    // of 32-row half qh at qh * 4 KiB, holding the stored block (qh, key half
    // wh) of the dS tile with the 16-byte chunks of each 1 KiB run permuted
    // by dst_lds_chunk (as in the dQ kernel).  Transposing-read addresses for
    // block t (tile t / 2, half t % 2) in stage 0; k step ks of the half adds
    // 256 (ks & 1) + 2048 (ks >> 1) bytes, stage st adds st * F_STH.
    // (the read offset field holds 16 bits: stages 2 and 3 read through a
    // second set of bases, 64 KiB up)
    uint32_t tra[2][TQ][2];
#pragma unroll
    for (int t = 0; t < TQ; ++t)
#pragma unroll
        for (int h4 = 0; h4 < 2; ++h4) {
            const int c = (t & 1) * 256 + hh * 64 + 32 * (t16 & 1) + g * 8 + h4 * 4 + s4;
            tra[0][t][h4] = lds_addr(smem) + (uint32_t)((t >> 1) * F_HB + dst_lds_chunk(c) * 16 + ((t16 >> 1) & 1) * 8);
            tra[1][t][h4] = tra[0][t][h4] + 2 * F_STH;
        }
    static_assert(2 * F_STH == 65536, "stage bases");
    // wave w copies the 64-key half of tile i0 + w (zeros when the tile has
    // no slot: past the last row tile, or above the diagonal)
    const int iw = i0 + w;
    auto stage = [&](int jh, int st) {
        const int jt = jh >> 1, wh = jh & 1;
        const bool ok = iw < tr_count && jt <= iw / 2;
        const __amdgpu_buffer_rsrc_t r =
            make_rsrc(dSw + dst_tile(bh, ok ? iw : 0, ok ? jt : 0, tr_count, tc, true), ok ? F_DS_B : 0);
#pragma unroll
        for (int k = 0; k < F_HB / 1024; ++k) {
            const int qh = k >> 2, run = k & 3;
            bdma16_l2(r, dst_lds_chunk((2 * qh + wh) * 256 + run * 64 + lane) * 16,
                      smem + st * F_STH + w * F_HB + qh * 4096 + run * 1024);
        }
    };
    // the wave's K image slice of key half jh: 16-key steps 4 (jh & 1) ..
    const uint32_t kvo = (uint32_t)((db * (BC / 16) * 64 + lane) * 16);
    auto load_k = [&](int jh, bf16x8* kb) {
        const __bf16* kt = Kimg + kimg_tile(bh, jh >> 1, tc, HD);
        static_for<0, KH>([&](auto ksI) {
            constexpr int ks = decltype(ksI)::value;
            gload16_l2<ks * 1024>(kb[ks], kt, kvo + (jh & 1) * 4096);
        });
    };

    bf16x8 kb[F_NST][KH];
    f32x16 acc[TQ];
#pragma unroll
    for (int t = 0; t < TQ; ++t) acc[t] = zero16();
    // steps 0 .. F_NST - 2 in flight before the first; a step past the end
    // reloads the last one, so every step issues the same loads
    static_for<0, F_NST - 1>([&](auto sI) {
        constexpr int s0 = decltype(sI)::value;
        stage(min(s0, nh - 1), s0);
        load_k(min(s0, nh - 1), kb[s0]);
    });
    auto step = [&](int jh, auto stI) {
        constexpr int st = decltype(stI)::value;
        constexpr int nx = (st + F_NST - 1) % F_NST;     // the stage of step jh + F_NST - 1
        // this step's loads have landed (the F_NST - 2 later steps' remain)
        vm_wait4<(F_NST - 2) * F_STEP_VM>(kb[st]);
        __builtin_amdgcn_s_barrier();           // landed for every wave; stage nx is free
        stage(min(jh + F_NST - 1, nh - 1), nx);
        load_k(min(jh + F_NST - 1, nh - 1), kb[nx]);
        if (jh >= nh) return;
        // A operands: the step's first k step is read up front; after each
        // product (ks, t) the reads of (ks + 1, t) are issued, so that 14
        // reads (7 products' worth) are in flight behind the one waited for
        u32x2 ta[KH][TQ][2];
        auto rd = [&](auto ksI, auto tI) {
            constexpr int ks = decltype(ksI)::value, t = decltype(tI)::value;
            constexpr int off = (st & 1) * F_STH + 256 * (ks & 1) + 2048 * (ks >> 1);
            tr_read2o<off>(ta[ks][t][0], ta[ks][t][1], tra[st >> 1][t][0], tra[st >> 1][t][1]);
        };
        static_for<0, TQ>([&](auto tI) { rd(std::integral_constant<int, 0>{}, tI); });
        static_for<0, KH>([&](auto ksI) {
            constexpr int ks = decltype(ksI)::value;
            static_for<0, TQ>([&](auto tI) {
                constexpr int t = decltype(tI)::value;
                // issued after (ks, t): (ks, t + 1 ..) and, but for the last
                // k step, (ks + 1, .. t - 1)
                lgkm_wait<ks + 1 < KH ? 2 * (TQ - 1) : 2 * (TQ - 1 - t)>(ta[ks][t][0], ta[ks][t][1]);
                acc[t] = mfma32(cat_u(ta[ks][t][0], ta[ks][t][1]), kb[st][ks], acc[t]);
                if constexpr (ks + 1 < KH) rd(std::integral_constant<int, ks + 1>{}, tI);
            });
        });
    };
    for (int jh = 0; jh < nh; jh += F_NST) {
        step(jh, std::integral_constant<int, 0>{});
        step(jh + 1, std::integral_constant<int, 1>{});
        step(jh + 2, std::integral_constant<int, 2>{});
        step(jh + 3, std::integral_constant<int, 3>{});
    }
    vm_wait4<0>(kb[0]);                          // no copy into LDS outlives the phase

    // ---- dQ = scale * acc, bf16, through a buffer resource over the rows
    //      [i0 * 64, q_end): element r of block t is row 32 t + 8 (r / 4) +
    //      4 g + r % 4 of the item's rows, column 32 db + lane % 32
    const int l32 = lane & 31;
    const int q0u = __builtin_amdgcn_readfirstlane(i0 * BR);
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(dQ + (size_t)bh * N * HD + (size_t)q0u * HD,
                  __builtin_amdgcn_readfirstlane(max(0, q_end - q0u) * HD * 2));
    const int vo = (4 * g * HD + db * 32 + l32) * 2;
#pragma unroll
    for (int t = 0; t < TQ; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int so = (t * 32 + 8 * (r >> 2)) * HD * 2;
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(short, (__bf16)(acc[t][r] * scale)), rq,
                                                  vo + (r & 3) * HD * 2, so, 0);
        }
    }
    __syncthreads();                             // every wave is done with the stages
}

// wave-uniform copies of a call's arguments (a call passes them in vector
// registers)
template <typename T>
__device__ __forceinline__ T* uni(T* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float uni(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

struct FusedArgs {
    const __bf16* Q;
    const __bf16* K;
    const __bf16* V;
    const __bf16* dO;
    const float* Lb;
    const float* Dp;
    __bf16* dSw;
    __bf16* Kimg;
    __bf16* dQ;
    __bf16* dK;
    __bf16* dV;
    int* ctrl;
    float* part;                                 // G > 1: fp32 dK / dV partials, one per query head
    int BH, H, G, N, n_pad;
    float scale;
};

// Claim the next ticket of queue q (wave 0 lane 0; broadcast through LDS)
// and decode it: returns false once the queue is exhausted; `valid` is false
// for the missing second head of an odd last pair.
__device__ __forceinline__ bool fused_claim(char* smem, const FusedArgs& a, int q, int wave, int& bh, int& j,
                                            bool& valid) {
    int* const ticket = reinterpret_cast<int*>(smem + FusedSmem::ticket);
    const int tc2 = (a.N + BC2 - 1) / BC2;
    const int nq = q < a.BH ? (a.BH - q + 7) / 8 : 0;       // heads q, q + 8, ...
    const int n_items = (nq + 1) / 2 * 2 * tc2;
    if (wave == 0 && lane_here() == 0)
        *ticket = __hip_atomic_fetch_add(a.ctrl + q, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int t = __builtin_amdgcn_readfirstlane(*ticket);
    __syncthreads();                             // read by every wave before the slot is reused
    if (t >= n_items) return false;
    const int p = t / (2 * tc2), r = t % (2 * tc2);
    const int lh = 2 * p + (r & 1);
    valid = lh < nq;
    bh = q + 8 * lh;
    j = r / 2;
    return true;
}

// One item: the dK/dV loop of key tile j of head bh (publishing its
// progress), then, once every item j' < j of the head has stored the dS
// tiles of query tiles 4 j .. 4 j + 3, the dQ of those tiles.  GQA: bh is a
// query head of a group of G > 1 sharing one K / V head.
template <bool GQA>
__device__ __forceinline__ void fused_item(char* smem, const FusedArgs& a, int bh, int j, int wave) {
    const int tc2 = (a.N + BC2 - 1) / BC2;
    int* const st = reinterpret_cast<int*>(smem + FusedSmem::state);
    if (wave == 0 && lane_here() == 0) {
        const uint64_t slot = reinterpret_cast<uint64_t>(a.ctrl + F_CTRL + (size_t)bh * tc2 + j);
        st[4] = (int)(uint32_t)slot;
        st[5] = (int)(uint32_t)(slot >> 32);
    }
    __syncthreads();
    if constexpr (GQA) {
        // query head bh is row (K / V head, part = its index in the group) of
        // a dK/dV grid with one part per query head; its dK and dV go out as
        // fp32 partials, which gqa_reduce_kernel sums over the group
        const int G = here_s(a.G), H = a.H;
        const int mapped = ((bh / H) * (H / G) + (bh % H) / G) * G + (bh % H) % G;
        dkdv_w64_item<true, true>(smem, a.Q, a.K, a.V, a.dO, a.Lb, a.Dp, a.dSw, a.Kimg, a.dK, a.dV, a.BH, H, G,
                                  G, a.part, a.N, a.n_pad, a.scale, mapped, j, nullptr, wave);
    } else {
        dkdv_w64_item<true, true>(smem, a.Q, a.K, a.V, a.dO, a.Lb, a.Dp, a.dSw, a.Kimg, a.dK, a.dV, a.BH, a.H, 1,
                                  1, nullptr, a.N, a.n_pad, a.scale, bh, j, nullptr, wave);
    }
    // its own stores are complete: the loop ended in a barrier after
    // waiting for them
    if (wave == 0 && lane_here() == 0) {
        const int* prog = a.ctrl + F_CTRL + (size_t)bh * tc2;
        int spins = 0;
        for (int jp = 0; jp < j; ++jp) {
            while (__hip_atomic_load(prog + jp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) > 4 * j) {
                __builtin_amdgcn_s_sleep(2);
                if (++spins >= F_WAIT_LIMIT) {
                    __hip_atomic_store(a.ctrl + 9, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
        }
    }
    __syncthreads();
    fused_dq_phase(smem, a.Kimg, a.dSw, a.dQ, bh, 4 * j, a.N, a.scale, wave);
}

// Persistent (B200 attention blog, Chapter 14 "Persistent"): about one
// workgroup per CU, each claiming tickets of its XCD's queue one after
// another until the queue is empty.  An item only waits for items with
// smaller tickets of the same queue, which some workgroup claimed earlier and
// runs (or has finished), so every wait ends.  The workgroups check in as
// they exit (ctrl[8]).  GQA: the items are query heads of groups sharing a
// K / V head (dK / dV as fp32 partials).
template <bool GQA>
__global__ __attribute__((amdgpu_flat_work_group_size(NW2 * 64, NW2 * 64), amdgpu_waves_per_eu(1, 1)))
void bwd_fused_kernel(FusedArgs args) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int wave = wave_id();
    const int q = xcc_id();
    for (;;) {
        int bh = 0, j = 0;
        bool valid = false;
        if (!fused_claim(smem, args, q, here_s(wave), bh, j, valid)) break;
        if (valid) fused_item<GQA>(smem, args, bh, j, here_s(wave));
    }
    if (wave == 0 && lane_here() == 0)
        __hip_atomic_fetch_add(args.ctrl + 8, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Runs after bwd_fused_kernel, as one workgroup: any ticket still unclaimed
// (a queue whose XCD got no workgroup of the kernel, on a device whose
// workgroups are not dealt to all eight XCDs) is taken here, in queue order,
// so its items' reads of dS see either this workgroup's own stores or those
// of the kernel before (complete at the kernel boundary).  Normally every
// queue is already exhausted and this returns at once.  The item runs behind
// a call so that the loop does not hold its registers.
template <bool GQA>
__device__ __noinline__ void fused_item_call(char* smem, const FusedArgs* a, int bh, int j, int wave) {
    FusedArgs u;
    u.Q = uni(a->Q); u.K = uni(a->K); u.V = uni(a->V); u.dO = uni(a->dO); u.Lb = uni(a->Lb); u.Dp = uni(a->Dp);
    u.dSw = uni(a->dSw); u.Kimg = uni(a->Kimg); u.dQ = uni(a->dQ); u.dK = uni(a->dK); u.dV = uni(a->dV);
    u.ctrl = uni(a->ctrl); u.part = uni(a->part); u.BH = uni(a->BH); u.H = uni(a->H); u.G = uni(a->G);
    u.N = uni(a->N); u.n_pad = uni(a->n_pad);
    u.scale = uni(a->scale);
    fused_item<GQA>(uni(smem), u, uni(bh), uni(j), uni(wave));
}

template <bool GQA>
__global__ __attribute__((amdgpu_flat_work_group_size(NW2 * 64, NW2 * 64), amdgpu_waves_per_eu(1, 1)))
void bwd_fused_sweep_kernel(FusedArgs args) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int wave = wave_id();
    for (int q = 0; q < 8; ++q) {
        int bh = 0, j = 0;
        bool valid = false;
        while (fused_claim(smem, args, q, wave, bh, j, valid)) {
            if (!valid) continue;
            if (wave == 0 && lane_here() == 0)
                __hip_atomic_fetch_add(args.ctrl + 10, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            fused_item_call<GQA>(smem, &args, bh, j, wave);
        }
    }
}

}  // namespace bwd

// ----------------------------------------------------------------------------
// Host launchers
// ----------------------------------------------------------------------------
static int grid_for(long long items, int per_block, int cap) {
    long long b = (items + per_block - 1) / per_block;
    if (b < 1) b = 1;
    if (b > cap) b = cap;
    return (int)b;
}

hipError_t launch_bwd_preprocess(const void* o, const void* dO, float* D, int BH, int N, int d,
                                 hipStream_t stream) {
    const long long rows = (long long)BH * N;
    if (rows == 0) return hipSuccess;
    if (d == 512) {
        hipLaunchKernelGGL(bwd_preprocess_kernel<512>, dim3(grid_for(rows, 4, 8192)), dim3(256), 0,
                           stream, (const __bf16*)o, (const __bf16*)dO, D, rows);
    } else if (d == 128) {
        hipLaunchKernelGGL(bwd_preprocess_kernel<128>, dim3(grid_for(rows, 16, 8192)), dim3(256), 0,
                           stream, (const __bf16*)o, (const __bf16*)dO, D, rows);
    } else {
        hipLaunchKernelGGL(bwd_preprocess_kernel<64>, dim3(grid_for(rows, 32, 8192)), dim3(256), 0,
                           stream, (const __bf16*)o, (const __bf16*)dO, D, rows);
    }
    return hipGetLastError();
}

// Workspace, in order (each part 256-byte aligned): Lb and Dp (BH x n_pad
// fp32 each), the dS tiles (BH x dst_tiles_per_head x (BC x BR) bf16: the
// lower triangle when causal), the K image (BH / G x T_c x (BC x d) bf16) and,
// only when a group's query heads are split over NS > 1 workgroups, the
// grouped-query partials (2 x NS x BH / G x N x d fp32).  Every byte that is
// read is written earlier in the same call.
static size_t n_pad_of(int N) { return (size_t)((N + bwd::BR - 1) / bwd::BR) * bwd::BR; }
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// key tiles per K / V head of the dK/dV grid
static int dkdv_tiles(int N, int d) {
    if (d == 128) return (N + bwd::BC2 - 1) / bwd::BC2;
    return (N + bwd::BC - 1) / bwd::BC;
}

// Parts the G query heads of a group are split over: 1 (all in one
// workgroup, no partials) unless that leaves fewer than about six workgroups
// per CU, in which case the smallest divisor of G that reaches that.
static int gqa_parts(int BHkv, int N, int d, int G) {
    const long long rows = (long long)BHkv * dkdv_tiles(N, d);
    int ns = 1;
    while (ns < G && rows * ns < 1536) {
        int nx = ns + 1;
        while (G % nx) ++nx;
        ns = nx;
    }
    return ns;
}

struct WsLayout {
    size_t ctrl, lb, dp, ds, kimg, part, total;
    int n_ctrl;                                  // ints of the fused kernel's control block (0: none)
};

// The fused causal kernel serves d = 128; with grouped-query heads its items
// are the query heads, each writing fp32 dK / dV partials (one part per query
// head) that gqa_reduce_kernel sums over the group.
static bool use_fused(int G, int d, bool causal) { (void)G; return causal && d == 128; }

static WsLayout ws_layout(int BH, int G, int N, int d, bool causal) {
    WsLayout w{};
    const size_t rows = (size_t)BH * n_pad_of(N);
    const int tr = (N + bwd::BR - 1) / bwd::BR, tc = (N + bwd::BC - 1) / bwd::BC;
    const bool fused = use_fused(G, d, causal);
    const int ns = fused ? G : gqa_parts(BH / G, N, d, G);
    size_t o = 0;
    w.n_ctrl = fused ? bwd::F_CTRL + BH * ((N + bwd::BC2 - 1) / bwd::BC2) : 0;
    w.ctrl = o; o = align256(o + (size_t)w.n_ctrl * sizeof(int));
    w.lb = o;   o = align256(o + rows * sizeof(float));
    w.dp = o;   o = align256(o + rows * sizeof(float));
    w.ds = o;   o = align256(o + (size_t)BH * bwd::dst_tiles_per_head(tr, tc, causal) * bwd::DST_EL * 2);
    // K images: one per K / V head; the fused kernel keeps one per query head
    w.kimg = o; o = align256(o + (size_t)(fused ? BH : BH / G) * tc * bwd::BC * d * 2);
    w.part = o; o = align256(o + (ns > 1 ? 2 * (size_t)ns * (BH / G) * N * d * sizeof(float) : 0));
    w.total = o;
    return w;
}

size_t bwd_workspace_bytes(int BH, int G, int N, int d, bool causal) {
    return ws_layout(BH, G, N, d, causal).total;
}

// BHkv = B * H / G key / value heads (the dK/dV grid has BHkv * ns rows)
template <int HD, bool CAUSAL>
static hipError_t launch_dkdv(const void* q, const void* k, const void* v, const void* dO,
                              const float* Lb, const float* Dp, __bf16* dSw, __bf16* kimg, void* dk,
                              void* dv, int BHkv, int H, int G, int ns, float* part, int N, int n_pad,
                              float scale, hipStream_t stream) {
    if constexpr (HD == 128) {
        using S2 = bwd::Smem2;
        auto kern = bwd::bwd_dkdv_w64_kernel<CAUSAL>;
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, S2::bytes);
        if (e != hipSuccess) return e;
        const int tc2 = (N + bwd::BC2 - 1) / bwd::BC2;
        hipLaunchKernelGGL(kern, dim3(BHkv * ns * tc2), dim3(bwd::NW2 * 64), S2::bytes, stream,
                           (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)dO,
                           Lb, Dp, dSw, kimg, (__bf16*)dk, (__bf16*)dv, BHkv * ns, H, G, ns, part, N,
                           n_pad, scale);
        return hipGetLastError();
    } else {
        using S = bwd::Smem<HD>;
        auto kern = bwd::bwd_dkdv_kernel<HD, CAUSAL>;
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, S::bytes);
        if (e != hipSuccess) return e;
        const int tc = (N + bwd::BC - 1) / bwd::BC;
        hipLaunchKernelGGL(kern, dim3(BHkv * ns * tc), dim3(bwd::NT), S::bytes, stream, (const __bf16*)q,
                           (const __bf16*)k, (const __bf16*)v, (const __bf16*)dO, Lb, Dp, dSw, kimg,
                           (__bf16*)dk, (__bf16*)dv, BHkv * ns, H, G, ns, part, N, n_pad, scale);
        return hipGetLastError();
    }
}

template <int HD, bool CAUSAL>
static hipError_t launch_dq(const __bf16* kimg, const __bf16* dSw, void* dq, int BH, int H, int G,
                            int N, float scale, hipStream_t stream) {
    const int tr = (N + bwd::BR - 1) / bwd::BR;
    hipLaunchKernelGGL((bwd::bwd_dq_kernel<HD, CAUSAL>), dim3(BH * ((tr + 1) / 2)), dim3(bwd::QW * 64), 0, stream,
                       kimg, dSw, (__bf16*)dq, BH, H, G, N, scale);
    return hipGetLastError();
}

template <int HD, bool CAUSAL>
static hipError_t launch_pair(const void* q, const void* k, const void* v, const void* dO,
                              const float* Lb, const float* Dp, __bf16* dSw, __bf16* kimg, float* part,
                              void* dq, void* dk, void* dv, int BH, int H, int G, int N, int n_pad,
                              float scale, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    const int ns = gqa_parts(BH / G, N, HD, G);
    hipError_t e;
    if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return e;
    e = launch_dkdv<HD, CAUSAL>(q, k, v, dO, Lb, Dp, dSw, kimg, dk, dv, BH / G, H, G, ns, part, N, n_pad,
                                scale, stream);
    if (e != hipSuccess) return e;
    if (ev1 && (e = hipEventRecord(ev1, stream)) != hipSuccess) return e;
    if (ns > 1) {
        const long long n = (long long)(BH / G) * N * HD;
        hipLaunchKernelGGL(gqa_reduce_kernel, dim3(grid_for(2 * n, 1024, 16384)), dim3(256), 0, stream,
                           part, (__bf16*)dk, (__bf16*)dv, ns, n);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return launch_dq<HD, CAUSAL>(kimg, dSw, dq, BH, H, G, N, scale, stream);
}

// BH query heads, G of them per K / V head (G > 1: fp32 partials in `part`,
// summed after the fused kernel)
static hipError_t launch_fused(const void* q, const void* k, const void* v, const void* dO,
                               const float* Lb, const float* Dp, __bf16* dSw, __bf16* kimg, int* ctrl,
                               float* part, void* dq, void* dk, void* dv, int BH, int H, int G, int N,
                               int n_pad, float scale, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    const void* main_kern = G > 1 ? (const void*)bwd::bwd_fused_kernel<true> : (const void*)bwd::bwd_fused_kernel<false>;
    const void* sweep_kern =
        G > 1 ? (const void*)bwd::bwd_fused_sweep_kernel<true> : (const void*)bwd::bwd_fused_sweep_kernel<false>;
    for (const void* kern : {main_kern, sweep_kern}) {
        hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bwd::FusedSmem::bytes);
        if (e != hipSuccess) return e;
    }
    bwd::FusedArgs a{(const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)dO, Lb, Dp, dSw, kimg,
                     (__bf16*)dq, (__bf16*)dk, (__bf16*)dv, ctrl, G > 1 ? part : nullptr, BH, H, G, N,
                     n_pad, scale};
    // one workgroup per CU (LDS allows no more), as many per XCD as the
    // largest queue has items at most; queue 0 holds the most heads
    // (ceil(BH / 8)), taken in pairs
    const int tc2 = (N + bwd::BC2 - 1) / bwd::BC2;
    const int nq0 = (BH + 7) / 8;
    const int per_xcd = (nq0 + 1) / 2 * 2 * tc2;
    hipError_t e;
    int dev = 0, cus = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    const int grid = std::min(8 * per_xcd, std::max(8, cus / 8 * 8));
    if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return e;
    if (G > 1)
        hipLaunchKernelGGL(bwd::bwd_fused_kernel<true>, dim3(grid), dim3(bwd::NW2 * 64), bwd::FusedSmem::bytes, stream, a);
    else
        hipLaunchKernelGGL(bwd::bwd_fused_kernel<false>, dim3(grid), dim3(bwd::NW2 * 64), bwd::FusedSmem::bytes, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (G > 1)
        hipLaunchKernelGGL(bwd::bwd_fused_sweep_kernel<true>, dim3(1), dim3(bwd::NW2 * 64), bwd::FusedSmem::bytes, stream, a);
    else
        hipLaunchKernelGGL(bwd::bwd_fused_sweep_kernel<false>, dim3(1), dim3(bwd::NW2 * 64), bwd::FusedSmem::bytes, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ev1 && (e = hipEventRecord(ev1, stream)) != hipSuccess) return e;
    if (G > 1) {
        const long long n = (long long)(BH / G) * N * 128;
        hipLaunchKernelGGL(gqa_reduce_kernel, dim3(grid_for(2 * n, 1024, 16384)), dim3(256), 0, stream,
                           part, (__bf16*)dk, (__bf16*)dv, G, n);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                      const float* D, void* dq, void* dk, void* dv, void* workspace, int BH, int H,
                      int G, int N, int d, bool causal, float scale, hipStream_t stream,
                      hipEvent_t main_start, hipEvent_t main_stop) {
    if ((long long)BH * N == 0) return hipSuccess;
    const int n_pad = (int)n_pad_of(N);
    const size_t rows = (size_t)BH * n_pad;
    const WsLayout w = ws_layout(BH, G, N, d, causal);
    char* ws = (char*)workspace;
    int* ctrl = (int*)(ws + w.ctrl);
    float* Lb = (float*)(ws + w.lb);
    float* Dp = (float*)(ws + w.dp);
    __bf16* dSw = (__bf16*)(ws + w.ds);
    __bf16* kimg = (__bf16*)(ws + w.kimg);
    float* part = (float*)(ws + w.part);
    hipLaunchKernelGGL(bwd_prep_kernel, dim3(grid_for((long long)rows, 256, 4096)), dim3(256), 0,
                       stream, Lb, Dp, lse, D, BH, N, n_pad, ctrl, w.n_ctrl, bwd::F_CTRL);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (use_fused(G, d, causal))
        return launch_fused(q, k, v, dO, Lb, Dp, dSw, kimg, ctrl, part, dq, dk, dv, BH, H, G, N, n_pad, scale,
                            stream, main_start, main_stop);
    if (d == 128)
        return causal ? launch_pair<128, true>(q, k, v, dO, Lb, Dp, dSw, kimg, part, dq, dk, dv, BH, H, G, N, n_pad, scale, stream, main_start, main_stop)
                      : launch_pair<128, false>(q, k, v, dO, Lb, Dp, dSw, kimg, part, dq, dk, dv, BH, H, G, N, n_pad, scale, stream, main_start, main_stop);
    return causal ? launch_pair<64, true>(q, k, v, dO, Lb, Dp, dSw, kimg, part, dq, dk, dv, BH, H, G, N, n_pad, scale, stream, main_start, main_stop)
                  : launch_pair<64, false>(q, k, v, dO, Lb, Dp, dSw, kimg, part, dq, dk, dv, BH, H, G, N, n_pad, scale, stream, main_start, main_stop);
}

}  // namespace attn
