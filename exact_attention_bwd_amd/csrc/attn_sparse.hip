// Top-k sparse attention for gfx950: every query row i attends to the keys its
// index list I_i names, and all query heads of a group share one K/V head.
//
// The method is the DSA (top-k sparse) attention of cudnn-frontend PR #684
// ("Improve performance of SM100 DSA backward kernel"): for each query row
// the K and V rows of its index list are gathered and the dense attention
// formulas of "Writing Speed-of-Light Attention Backward Kernel for 5090 in
// CUDA" ("Mathematical Formulation") are applied to that set; dK and dV are
// summed over the heads and over every query row that selected the key.
// Head dims are fixed at d_qk = 576, d_v = 512; query heads come in groups of
// 64 (the M dimension of every product, as in the PR's design).
//
// CDNA4 mapping:
//  * one workgroup per (query row, group of 64 heads): 4 wave64s, one per
//    SIMD, in the forward and the dQ kernel; 8 (two per SIMD) in the backward
//    per-row kernel, so that one wave's MFMAs cover another's gather loads.
//  * the gathered K rows feed the score products straight from memory (each
//    lane's 16 bytes are one row-contiguous MFMA operand); V rows, Q_i, dO_i
//    and K chunks that are read with a transposing LDS read are copied into
//    LDS by per-lane-addressed buffer -> LDS copies, i.e. the gather itself.
//  * dK and dV: the PR adds every row's contribution into fp32 buffers with
//    atomics.  fp32 atomics on this GPU run at about 1.3 TB/s of payload
//    wherever the target lives (in or out of L2, any scope), and a 4096-row,
//    top-512 problem needs 9.1 GB of them.  Instead the per-row kernel stores
//    each (row, slot)'s contribution (summed over the head group) with plain
//    stores, a counting-sort transpose of the index lists gives every key its
//    list of (row, slot) pairs in row order, and a reduction kernel sums them
//    per key in that fixed order, in fp32.
//  * a stored contribution is fp16 times a power of two chosen per (row, slot)
//    and per part (dV, dK) from a bound on its magnitude, so it cannot
//    overflow and keeps fp16's 11-bit significand: a relative error of at most
//    2^-12 per stored value, 8x below the bf16 rounding of the output, at half
//    the bytes of fp32.
//  * dQ = scale * dS K_I needs dS with one head per lane, so the per-row
//    kernel stores dS (bf16, as the PR rounds it for its dQ product) and a
//    second per-row kernel forms dQ in registers, as in the dense backward.
#include "asm_ops.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace attn {
namespace sp {

constexpr int DQK = 576;
constexpr int DV = 512;
constexpr int HG = 64;                 // query heads per workgroup
constexpr int QROW = 1280;             // LDS row stride (bytes) of a 576-wide bf16 row
constexpr int VROW = 1024;             // LDS row stride (bytes) of a 512-wide bf16 row
constexpr int PW = DV + DQK;           // fp16 values of one (row, slot) dK/dV contribution
constexpr int RB = 16;                 // query rows per block of the index transpose
constexpr int MAX_NKV = 16384;         // keys the transpose can count in LDS
constexpr int SBW_WAVES = 8;           // waves of the per-row backward kernel
constexpr int SBW_CHUNK = SBW_WAVES * 32;   // slots per chunk of that kernel
constexpr int kDropOffset = 0x40000000;    // buffer offset past any contribution block
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// LDS rows start on a 256-byte bank line; the 16-byte chunk c of row r is
// stored at chunk (c & ~15) | ((c & 15) ^ lswz(r)).  For any 16 consecutive
// rows lswz takes 16 distinct values, so 16-byte reads of one chunk across 16
// rows are conflict-free; its bits 2..3 are r & 3, so a transposing read (4
// rows x 4 chunks) is conflict-free too.
__device__ __forceinline__ int lswz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ int lchunk(int r, int c) { return (c & ~15) | ((c & 15) ^ lswz(r)); }

// byte offset of element `col` (a multiple of 4) of row r in a swizzled tile
template <int STRIDE>
__device__ __forceinline__ int loff(int r, int col) {
    return r * STRIDE + lchunk(r, col >> 3) * 16 + (col & 7) * 2;
}

// dS^T rows (one slot, 64 heads = 128 bytes): the 8-byte unit u (4 heads) of
// slot row s lives at unit u ^ tswz(s); the same argument as above on 8-byte
// units makes the transposing reads of 4 slots x 4 units conflict-free.
__device__ __forceinline__ int tswz(int s) { return ((s & 3) << 2) | ((s >> 2) & 3); }

__device__ __forceinline__ int dsoff(int s, int u) {       // element offset
    return s * HG + ((u ^ tswz(s)) << 2);
}

__device__ __forceinline__ int valid_slots(const int* tlen, int i, int topk) {
    if (!tlen) return topk;
    const int n = tlen[i];
    return n < 0 ? 0 : (n > topk ? topk : n);
}

// key of slot s of row i, or -1 when the slot is absent (past the row's
// length, negative, or not a key index)
__device__ __forceinline__ int slot_key(const int* irow, int s, int nval, int Nkv) {
    if (s >= nval) return -1;
    const int k = irow[s];
    return (k >= 0 && k < Nkv) ? k : -1;
}

// Copy one 576-wide bf16 row (1152 bytes, from a descriptor whose record
// holds that row at byte `src`) into swizzled LDS row r: 64 lanes cover
// chunks 0..63, 16 lanes the last bank line (chunks 64..79, of which 72..79 are
// padding and read as zero because they lie past the descriptor's end).
__device__ __forceinline__ void stage_qrow(__amdgpu_buffer_rsrc_t rs, int src, char* tile, int r,
                                           int lane) {
    bdma16(rs, src + lchunk(r, lane) * 16, tile + r * QROW);
    if (lane < 16) bdma16(rs, src + (64 + (lane ^ lswz(r))) * 16, tile + r * QROW + 1024);
}

__device__ __forceinline__ void stage_vrow(__amdgpu_buffer_rsrc_t rs, int src, char* tile, int r,
                                           int lane) {
    bdma16(rs, src + lchunk(r, lane) * 16, tile + r * VROW);
}

// ----------------------------------------------------------------------------
// Forward: O = softmax(scale * Q_i K_I^T) V_I, L = log-sum-exp, per head, with
// the online softmax over 64-slot tiles (running max m and sum l per head,
// rescale by 2^(m_old - m_new)).  Wave (hb, vh) owns heads 32 hb .. + 31 of the
// group and output columns 256 vh .. + 255; it scores slots 32 vh .. + 31 of
// each tile, and the two waves of a head block swap their tile maxima and
// their P through LDS.  S^T = K Q^T puts one head per lane, so P^T is the B
// operand of O^T = V^T P^T directly; V^T comes from transposing reads of the
// gathered V tile, which is double-buffered one tile ahead.
// ----------------------------------------------------------------------------
struct FwdSmem {
    static constexpr int off_q = 0;                          // Q_i: 64 x QROW
    static constexpr int off_v = HG * QROW;                  // V tile: 64 slots x VROW
    static constexpr int off_m = off_v + 64 * VROW;          // float [4][64] tile maxima
    static constexpr int off_l = off_m + 4 * 64 * 4;         // float [4][64] tile sums
    static constexpr int off_p = off_l + 4 * 64 * 4;         // bf16x8 [4][2][64] P^T operands
    static constexpr int bytes = off_p + 4 * 2 * 64 * 16;
};

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void sfwd_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                 const __bf16* __restrict__ V, const int* __restrict__ idx,
                 const int* __restrict__ tlen, __bf16* __restrict__ O, float* __restrict__ Lse,
                 int Hq, int Nq, int Nkv, int topk, float scale) {
    using S = FwdSmem;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int lane = threadIdx.x & 63, w = wave_id();
    const int hb = w & 1, vh = w >> 1, pw = w ^ 2;   // partner: same heads, other half
    const int l32 = lane & 31, g = lane >> 5, t16 = lane & 15, hh = (lane >> 4) & 1, s4 = t16 >> 2;
    const int G = Hq / HG;
    const int logical = xcd_remap(blockIdx.x, Nq * G);
    const int i = logical / G, hg = logical % G;
    const int nval = valid_slots(tlen, i, topk);
    const int ntiles = (nval + 63) / 64;
    const int* irow = idx + (size_t)i * topk;
    const int head = hg * HG + hb * 32 + l32;    // this lane's head (accumulator column)

    const __amdgpu_buffer_rsrc_t krs = make_rsrc(K, Nkv * DQK * 2);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V, Nkv * DV * 2);
    char* const vt = smem + S::off_v;
    const char* const qt = smem + S::off_q;
    float* xm = reinterpret_cast<float*>(smem + S::off_m);
    float* xl = reinterpret_cast<float*>(smem + S::off_l);
    bf16x8* xp = reinterpret_cast<bf16x8*>(smem + S::off_p);

    // ---- Q_i of the group's 64 heads into LDS (rows 16 w .. + 15 per wave)
#pragma unroll 4
    for (int rr = 0; rr < 16; ++rr) {
        const int h = w * 16 + rr;
        const size_t hrow = (size_t)(hg * HG + h) * Nq + i;
        stage_qrow(make_rsrc(Q + hrow * DQK, DQK * 2), 0, smem + S::off_q, h, lane);
    }

    f32x16 acc[8];                               // O^T: 8 blocks of 32 columns x 32 heads
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[b] = zero16();
    float m = -__builtin_inff(), lsum = 0.f;
    const float sl2 = scale * kLog2e;

    for (int t = 0; t < ntiles; ++t) {
        // ---- gather V rows of the tile (wave w: rows 16 w .. + 15; absent
        //      slots read past the end of V, i.e. zeros); lands by barrier 1
        const int key_lane = slot_key(irow, t * 64 + lane, nval, Nkv);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int r = w * 16 + rr;
            int key = __builtin_amdgcn_readlane(key_lane, r);
            key = key < 0 ? Nkv : key;
            stage_vrow(vrs, key * (DV * 2), vt, r, lane);
        }
        if (t == 0) __syncthreads();              // Q_i landed
        // ---- S^T (this wave's 32 slots x 32 heads) = K_I Q^T over d_qk
        const int kk = __shfl(key_lane, 32 * vh + l32);
        const int kbase = (kk < 0 ? Nkv : kk) * (DQK * 2) + 16 * g;
        f32x16 s = zero16();
#pragma unroll
        for (int ks = 0; ks < DQK / 16; ++ks) {
            const bf16x8 a = __builtin_bit_cast(
                bf16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, kbase + 32 * ks, 0, 0));
            const bf16x8 b = *reinterpret_cast<const bf16x8*>(qt + loff<QROW>(hb * 32 + l32, 16 * ks + 8 * g));
            s = mfma32(a, b, s);
        }
        const uint64_t vmask = __ballot(key_lane >= 0);
        float mt = -__builtin_inff();
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int sl = 32 * vh + 8 * (r >> 2) + 4 * g + (r & 3);
            s[r] = ((vmask >> sl) & 1) ? s[r] * sl2 : -__builtin_inff();
            mt = fmaxf(mt, s[r]);
        }
        mt = wave_max_pair32(mt);
        xm[w * 64 + lane] = mt;
        __syncthreads();                          // 1: maxima visible, V tile landed
        // ---- common running max of the head over both halves, P, sums
        const float mn = fmaxf(m, fmaxf(mt, xm[pw * 64 + lane]));
        const float mu = (mn == -__builtin_inff()) ? 0.f : mn;
        const float alpha = __builtin_amdgcn_exp2f(m - mu);
        float ls = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s[r] = __builtin_amdgcn_exp2f(s[r] - mu);
            ls += s[r];
        }
        ls += __shfl_xor(ls, 32);
        const bf16x8 p0 = pack_c8(s, 0), p1 = pack_c8(s, 8);
        xp[(w * 2 + 0) * 64 + lane] = p0;
        xp[(w * 2 + 1) * 64 + lane] = p1;
        xl[w * 64 + lane] = ls;
        __syncthreads();                          // 2: partner's P and sum visible
        const bf16x8 q0 = xp[(pw * 2 + 0) * 64 + lane], q1 = xp[(pw * 2 + 1) * 64 + lane];
        lsum = lsum * alpha + ls + xl[pw * 64 + lane];
        m = mn;
        if (__ballot(alpha != 1.f)) {
#pragma unroll
            for (int b = 0; b < 8; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[b][r] *= alpha;
        }
        // ---- O^T += V^T P^T over all 64 slots (own half, then partner's)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int sh = half ? (vh ^ 1) : vh;
            const int r0 = 32 * sh + 4 * g + s4;
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const int col = 32 * (8 * vh + b) + 16 * hh + 4 * (t16 & 3);
#pragma unroll
                for (int k4 = 0; k4 < 2; ++k4) {
                    const int ra = r0 + 16 * k4;
                    const bf16x8 a = cat44(
                        lds_read_tr(reinterpret_cast<const __bf16*>(vt + loff<VROW>(ra, col))),
                        lds_read_tr(reinterpret_cast<const __bf16*>(vt + loff<VROW>(ra + 8, col))));
                    const bf16x8 bp = half ? (k4 ? q1 : q0) : (k4 ? p1 : p0);
                    acc[b] = mfma32(a, bp, acc[b]);
                }
            }
        }
        __syncthreads();                          // 3: V tile, P and maxima free
    }

    // ---- O = O^T / l (rows with no valid slot: O = 0, L = -inf)
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    __bf16* orow = O + ((size_t)head * Nq + i) * DV;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const int col0 = 32 * (8 * vh + b);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = acc[b][q * 4 + e] * inv;
            *reinterpret_cast<bf16x4*>(orow + col0 + 8 * q + 4 * g) = __builtin_convertvector(o, bf16x4);
        }
    }
    if (vh == 0 && g == 0) {
        const float mu = (m == -__builtin_inff()) ? 0.f : m;
        Lse[(size_t)head * Nq + i] = lsum > 0.f ? (mu + __log2f(lsum)) * kLn2 : -__builtin_inff();
    }
}

// ----------------------------------------------------------------------------
// Backward, per (query row, head group): recompute S = Q_i K_I^T, P, dP =
// dO_i V_I^T and dS; store dS (bf16) for the dQ kernel and each slot's dV and
// (unscaled) dK contribution, summed over the 64 heads, as scaled fp16 (the
// two powers of two go to `pscale`, see contrib_exp).  Eight waves
// (two per SIMD); wave w owns slots 32 w .. + 31 of every 256-slot chunk and
// all 64 heads: S and dP have
// one slot per lane, which is the A layout of P^T and dS^T for dV = P^T dO and
// dK = dS^T Q (k = heads); dO_i and Q_i sit in LDS for the whole row and are
// read row-wise (A operands of S, dP) and transposed (B operands of dV, dK).
// ----------------------------------------------------------------------------
struct BwdSmem {
    static constexpr int off_q = 0;                          // 64 x QROW
    static constexpr int off_do = off_q + HG * QROW;         // 64 x VROW
    static constexpr int off_l = off_do + HG * VROW;         // 64 floats (L log2 e)
    static constexpr int off_d = off_l + HG * 4;             // 64 floats (D)
    static constexpr int off_mq = off_d + HG * 4;            // 64 floats: max |Q_h,:|
    static constexpr int off_mdo = off_mq + HG * 4;          // 64 floats: max |dO_h,:|
    static constexpr int off_sc = off_mdo + HG * 4;          // per wave: [2][32] inverse scales
    static constexpr int bytes = off_sc + SBW_WAVES * 2 * 32 * 4;
};

// Power-of-two scale of a stored contribution whose entries are at most `b`
// in magnitude: the stored value is c * 2^-e in fp16 with 2^-e b <= 2^14, so
// it stays below fp16's largest finite value with a factor 4 to spare (enough
// for the bf16 rounding of P and dS and the fp32 sums behind c); e is kept
// >= -120 so that 2^e and 2^-e are normal floats.
__device__ __forceinline__ int contrib_exp(float b) {
    const int e = __builtin_amdgcn_frexp_expf(b) - 14;     // b < 2^(e + 14) for b > 0
    return e < -120 ? -120 : e;
}

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sbwd_main_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                      const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                      const float* __restrict__ Lse, const float* __restrict__ Dd,
                      const int* __restrict__ idx, const int* __restrict__ tlen,
                      __bf16* __restrict__ dsw, _Float16* __restrict__ part,
                      float2* __restrict__ pscale, int Hq, int Nq, int Nkv, int topk, int tpad,
                      float scale) {
    using S = BwdSmem;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int lane = threadIdx.x & 63, w = wave_id();
    const int l32 = lane & 31, g = lane >> 5, t16 = lane & 15, hh = (lane >> 4) & 1, s4 = t16 >> 2;
    const int G = Hq / HG;
    const int logical = xcd_remap(blockIdx.x, Nq * G);
    const int i = logical / G, hg = logical % G;
    const int nval = valid_slots(tlen, i, topk);
    const int nchunks = (nval + SBW_CHUNK - 1) / SBW_CHUNK;
    const int* irow = idx + (size_t)i * topk;
    const size_t rowg = (size_t)i * G + hg;      // (row, head group) index

    // ---- Q_i, dO_i of the 64 heads into LDS (rows 8 w .. + 7 per wave); L, D
#pragma unroll 4
    for (int rr = 0; rr < 8; ++rr) {
        const int h = w * 8 + rr;
        const size_t hrow = (size_t)(hg * HG + h) * Nq + i;
        stage_qrow(make_rsrc(Q + hrow * DQK, DQK * 2), 0, smem + S::off_q, h, lane);
        stage_vrow(make_rsrc(dO + hrow * DV, DV * 2), 0, smem + S::off_do, h, lane);
    }
    if (w == 0) {
        const size_t hrow = (size_t)(hg * HG + lane) * Nq + i;
        reinterpret_cast<float*>(smem + S::off_l)[lane] = Lse[hrow] * kLog2e;
        reinterpret_cast<float*>(smem + S::off_d)[lane] = Dd[hrow];
    }
    __syncthreads();
    // ---- max |Q_h,:| and max |dO_h,:| per head: 8 lanes per head, 9 (Q) and 8
    //      (dO) 16-byte chunks per lane, then a max over the 8 lanes
    {
        const int h = threadIdx.x >> 3, p = threadIdx.x & 7;
        auto chunk_max = [](const char* row, int c, float m) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(row + c * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                m = fmaxf(m, fabsf(__uint_as_float(v[e] << 16)));
                m = fmaxf(m, fabsf(__uint_as_float(v[e] & 0xffff0000u)));
            }
            return m;
        };
        float mq = 0.f, md = 0.f;
#pragma unroll
        for (int m = 0; m < DQK / 64; ++m) mq = chunk_max(smem + S::off_q + h * QROW, lchunk(h, p + 8 * m), mq);
#pragma unroll
        for (int m = 0; m < DV / 64; ++m) md = chunk_max(smem + S::off_do + h * VROW, lchunk(h, p + 8 * m), md);
#pragma unroll
        for (int x = 1; x < 8; x <<= 1) {
            mq = fmaxf(mq, __shfl_xor(mq, x));
            md = fmaxf(md, __shfl_xor(md, x));
        }
        if (p == 0) {
            reinterpret_cast<float*>(smem + S::off_mq)[h] = mq;
            reinterpret_cast<float*>(smem + S::off_mdo)[h] = md;
        }
    }
    __syncthreads();

    const __bf16* Qs = reinterpret_cast<const __bf16*>(smem + S::off_q);
    const __bf16* dOs = reinterpret_cast<const __bf16*>(smem + S::off_do);
    const float* Ls = reinterpret_cast<const float*>(smem + S::off_l);
    const float* Ds = reinterpret_cast<const float*>(smem + S::off_d);
    const float* MQs = reinterpret_cast<const float*>(smem + S::off_mq);
    const float* MDs = reinterpret_cast<const float*>(smem + S::off_mdo);
    float* scw = reinterpret_cast<float*>(smem + S::off_sc) + w * 64;   // [0..31] dV, [32..63] dK
    const char* Qb = smem + S::off_q;
    const char* dOb = smem + S::off_do;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(K, Nkv * DQK * 2);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V, Nkv * DV * 2);
    const float sl2 = scale * kLog2e;
    (void)Qs;
    (void)dOs;
    // this row's contribution block, and the v_perm selector that keeps
    // (own low, partner's low) on even lanes, (partner's high, own high) on odd
    const __amdgpu_buffer_rsrc_t prs = make_rsrc(part + rowg * topk * PW, topk * PW * 2);
    const int odd = l32 & 1;
    const uint32_t psel = odd ? 0x03020706u : 0x05040100u;

    for (int c = 0; c < nchunks; ++c) {
        const int slot = c * SBW_CHUNK + w * 32 + l32;            // this lane's slot
        const int key = slot_key(irow, slot, nval, Nkv);
        const uint64_t vmask = __ballot(key >= 0);               // bit l32 (g = 0 half)
        const int kbq = (key < 0 ? Nkv : key) * (DQK * 2) + 16 * g;
        const int kbv = (key < 0 ? Nkv : key) * (DV * 2) + 16 * g;

        // ---- S = Q_i K^T and dP = dO_i V^T: 64 heads x this wave's 32 slots
        f32x16 sc[2], dp[2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            sc[hb] = zero16();
            dp[hb] = zero16();
        }
        // gathered K / V operands in groups of 4 k steps, two groups in flight
        // ahead of the products (the sched barriers keep the compiler from
        // hoisting all 68 loads)
        constexpr int GK = 4, PF = 2;
        auto gload = [&](__amdgpu_buffer_rsrc_t rs, int base, int ks) {
            return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, base + 32 * ks, 0, 0));
        };
        constexpr int NG = (DQK + DV) / 16 / GK;
        bf16x8 gb[PF + 1][GK];
        auto gissue = [&](int grp, bf16x8* dst) {
#pragma unroll
            for (int e = 0; e < GK; ++e) {
                const int ks = grp * GK + e;
                dst[e] = ks < DQK / 16 ? gload(krs, kbq, ks) : gload(vrs, kbv, ks - DQK / 16);
            }
        };
#pragma unroll
        for (int g0 = 0; g0 < PF; ++g0) gissue(g0, gb[g0]);
#pragma unroll
        for (int grp = 0; grp < NG; ++grp) {
            const int ks0 = grp * GK;                              // 0..35 K, 36..67 V
            if (grp + PF < NG) gissue(grp + PF, gb[(grp + PF) % (PF + 1)]);
            bf16x8* gcur = gb[grp % (PF + 1)];
#pragma unroll
            for (int e = 0; e < GK; ++e) {
                const int ks = ks0 + e;
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    if (ks < DQK / 16) {
                        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                            Qb + loff<QROW>(hb * 32 + l32, 16 * ks + 8 * g));
                        sc[hb] = mfma32(a, gcur[e], sc[hb]);
                    } else {
                        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                            dOb + loff<VROW>(hb * 32 + l32, 16 * (ks - DQK / 16) + 8 * g));
                        dp[hb] = mfma32(a, gcur[e], dp[hb]);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // ---- P = exp(scale S - L) (0 for absent slots), dS = P (dP - D); the
        //      slot's bounds sum_h |P| max|dO_h| and sum_h |dS| max|Q_h|
        const bool live = key >= 0;
        bf16x8 pa[2][2], da[2][2];
        float bv = 0.f, bk = 0.f;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int h0 = hb * 32 + 8 * q + 4 * g;
                const f32x4 lv = *reinterpret_cast<const f32x4*>(Ls + h0);
                const f32x4 dd = *reinterpret_cast<const f32x4*>(Ds + h0);
                const f32x4 mq = *reinterpret_cast<const f32x4*>(MQs + h0);
                const f32x4 md = *reinterpret_cast<const f32x4*>(MDs + h0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = q * 4 + e;
                    const float p = live ? __builtin_amdgcn_exp2f(
                                               __builtin_fmaf(sc[hb][r], sl2, -lv[e]))
                                         : 0.f;
                    sc[hb][r] = p;
                    dp[hb][r] = p * (dp[hb][r] - dd[e]);
                    bv = __builtin_fmaf(p, md[e], bv);
                    bk = __builtin_fmaf(fabsf(dp[hb][r]), mq[e], bk);
                }
            }
            pa[hb][0] = pack_c8(sc[hb], 0);
            pa[hb][1] = pack_c8(sc[hb], 8);
            da[hb][0] = pack_c8(dp[hb], 0);
            da[hb][1] = pack_c8(dp[hb], 8);
        }
        // ---- dS^T (bf16) for the dQ kernel: this lane's slot row, 4 heads per unit
        {
            __bf16* drow = dsw + rowg * (size_t)tpad * HG;
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    f32x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = dp[hb][q * 4 + e];
                    const int u = 8 * hb + 2 * q + g;
                    *reinterpret_cast<bf16x4*>(drow + dsoff(slot, u)) = __builtin_convertvector(v, bf16x4);
                }
        }
        // ---- the slot's scales: the two lane halves hold the heads' halves of
        //      the bounds; inverse scales to LDS for the store layout below,
        //      the scales themselves to pscale for the reduction
        const int slot0 = c * SBW_CHUNK + w * 32;
        {
            bv += __shfl_xor(bv, 32);
            bk += __shfl_xor(bk, 32);
            const int ev = contrib_exp(bv), ek = contrib_exp(bk);
            if (g == 0) {
                scw[l32] = __builtin_amdgcn_ldexpf(1.f, -ev);
                scw[32 + l32] = __builtin_amdgcn_ldexpf(1.f, -ek);
                if (live)
                    pscale[rowg * topk + slot] =
                        make_float2(__builtin_amdgcn_ldexpf(1.f, ev), __builtin_amdgcn_ldexpf(1.f, ek));
            }
            // the reads below are this wave's own LDS writes: LDS requests of a
            // wave complete in order, so waiting for the writes suffices
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_wave_barrier();
        }
        // ---- dV and dK contributions of the 32 slots, 4 column blocks at a time:
        //      C[m = slot][n = column], k = the 64 heads.  Register r of half g
        //      holds slot 8 (r >> 2) + 4 g + (r & 3) at column l32; lanes 2m and
        //      2m + 1 swap one value of each register pair (r, r + 1) so that
        //      each lane stores two adjacent fp16 columns of one slot: the even
        //      lane slot 8 (r >> 2) + 4 g + (r & 3), the odd lane the next one.
        //      Stores go through a descriptor over this row's block with
        //      per-lane byte offsets fixed for the chunk; absent slots get an
        //      offset past the block's end, so their stores are dropped.
        f32x4 isc[4];                            // inverse scales of this lane's 16 slots
        auto load_isc = [&](int part_off) {
#pragma unroll
            for (int q = 0; q < 4; ++q) isc[q] = *reinterpret_cast<const f32x4*>(scw + part_off + 8 * q + 4 * g);
        };
        int voff[4][2];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const int sl = 8 * q + 2 * pp + 4 * g + odd;
                voff[q][pp] = ((vmask >> sl) & 1) ? (slot0 + sl) * (PW * 2) + 2 * (l32 - odd) : kDropOffset;
            }
        auto contrib = [&](const char* tile, int stride, bool is_v, int nblk, int blk0, int colbase) {
            f32x16 cacc[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) cacc[b] = zero16();
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int k4 = 0; k4 < 2; ++k4) {
                    const int hr = hb * 32 + 16 * k4 + 4 * g + s4;
#pragma unroll
                    for (int b = 0; b < 2; ++b) {
                        if (b < nblk) {
                            const int col = 32 * (blk0 + b) + 16 * hh + 4 * (t16 & 3);
                            const int o0 = stride == QROW ? loff<QROW>(hr, col) : loff<VROW>(hr, col);
                            const int o8 = stride == QROW ? loff<QROW>(hr + 8, col) : loff<VROW>(hr + 8, col);
                            const bf16x8 bop = cat44(lds_read_tr(reinterpret_cast<const __bf16*>(tile + o0)),
                                                     lds_read_tr(reinterpret_cast<const __bf16*>(tile + o8)));
                            cacc[b] = mfma32(is_v ? pa[hb][k4] : da[hb][k4], bop, cacc[b]);
                        }
                    }
                }
            const int coff = 2 * (colbase + 32 * blk0);       // uniform byte offset of the column block
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                if (b < nblk) {
#pragma unroll
                    for (int r = 0; r < 16; r += 2) {
                        // x = (slot r, slot r + 1) at this lane's column; y = the same of lane l ^ 1
                        const f16x2 hx = __builtin_convertvector(
                            (f32x2{cacc[b][r] * isc[r >> 2][r & 3], cacc[b][r + 1] * isc[r >> 2][(r & 3) + 1]}), f16x2);
                        const uint32_t x = __builtin_bit_cast(uint32_t, hx);
                        const uint32_t y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xb1, 0xf, 0xf, false);
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_amdgcn_perm(y, x, psel), prs,
                                                              voff[r >> 2][(r & 3) >> 1] + 64 * b, coff, 0);
                    }
                }
            }
        };
        load_isc(0);
#pragma unroll 1
        for (int blk = 0; blk < DV / 32; blk += 2) contrib(dOb, VROW, true, 2, blk, 0);
        load_isc(32);
#pragma unroll 1
        for (int blk = 0; blk < DQK / 32; blk += 2) contrib(Qb, QROW, false, 2, blk, DV);
    }
}

// ----------------------------------------------------------------------------
// dQ_i = scale * dS_i K_I per (query row, head group).  Chunks of 32 slots:
// the dS^T rows (stored by the kernel above in this LDS layout) and the
// gathered K rows are copied into a ring of DQ_NST LDS stages, two chunks
// ahead of the products; both operands come from transposing reads.  The
// row's keys are read once into LDS, so that no global load sits between the
// stage copies (a wait for it would wait for every copy issued before it).
// Wave w owns head block w & 1 and 9 of the 18 column blocks of d_qk.
// ----------------------------------------------------------------------------
constexpr int DQ_CH = 32;                        // slots per chunk
constexpr int DQ_DS = DQ_CH * HG * 2;            // bytes of dS^T per chunk (4 KiB)
constexpr int DQ_K = DQ_CH * QROW;               // bytes of K per chunk (40 KiB)
constexpr int DQ_STAGE = DQ_DS + DQ_K;
constexpr int DQ_NST = 3;                        // stages in the ring
constexpr int DQ_MAXT = 1024;                    // slots whose keys the LDS list holds
constexpr int DQ_KEYS = DQ_NST * DQ_STAGE;       // LDS offset of the key list
constexpr int DQ_SMEM = DQ_KEYS + DQ_MAXT * 4;
constexpr int DQ_STAGE_VM = 1 + 2 * 8;           // buffer -> LDS copies one stage issues per wave

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void sbwd_dq_kernel(const __bf16* __restrict__ K, const __bf16* __restrict__ dsw,
                    const int* __restrict__ idx, const int* __restrict__ tlen,
                    __bf16* __restrict__ dQ, int Hq, int Nq, int Nkv, int topk, int tpad,
                    float scale) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int lane = threadIdx.x & 63, w = wave_id();
    const int l32 = lane & 31, g = lane >> 5, t16 = lane & 15, hh = (lane >> 4) & 1, s4 = t16 >> 2;
    const int hb = w & 1, db0 = (w >> 1) * 9;
    const int G = Hq / HG;
    const int logical = xcd_remap(blockIdx.x, Nq * G);
    const int i = logical / G, hg = logical % G;
    const int nval = valid_slots(tlen, i, topk);
    const int nch = (nval + DQ_CH - 1) / DQ_CH;
    const int* irow = idx + (size_t)i * topk;
    const size_t rowg = (size_t)i * G + hg;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(K, Nkv * DQK * 2);
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(dsw + rowg * (size_t)tpad * HG, tpad * HG * 2);
    int* keys = reinterpret_cast<int*>(smem + DQ_KEYS);

    // keys of the row's slots s0 .. s0 + DQ_MAXT - 1 (Nkv for an absent slot:
    // a row past K's end, which the copies read as zeros)
    auto load_keys = [&](int s0) {
        for (int s = threadIdx.x; s < DQ_MAXT; s += 256) {
            const int k = slot_key(irow, s0 + s, nval, Nkv);
            keys[s] = k < 0 ? Nkv : k;
        }
    };
    // chunk c into stage buf: dS^T (4 x 1 KiB, one per wave), K rows 8 w .. + 7.
    // The loop's LDS reads are issued from assembly with explicit waits: the
    // compiler would otherwise wait for every copy in flight before each one.
    auto stage = [&](int c, int buf) {
        char* st = smem + buf * DQ_STAGE;
        bdma16(drs, c * DQ_DS + w * 1024 + lane * 16, st + w * 1024);
        u32x4 kv[2];
        const uint32_t ka = lds_addr(keys + (c * DQ_CH) % DQ_MAXT + w * 8);
        lds_ld<0>(kv[0], ka);
        lds_ld<16>(kv[1], ka);
        lgkm_wait<0>(kv[0], kv[1]);
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            const int key = __builtin_amdgcn_readfirstlane((int)kv[rr >> 2][rr & 3]);
            stage_qrow(krs, key * (DQK * 2), st + DQ_DS, w * 8 + rr, lane);
        }
    };

    f32x16 acc[9];
#pragma unroll
    for (int b = 0; b < 9; ++b) acc[b] = zero16();
    load_keys(0);
    __syncthreads();
    constexpr int CPL = DQ_MAXT / DQ_CH;         // chunks per key-list piece
    for (int c = 0; c < DQ_NST - 1 && c < nch && c < CPL; ++c) stage(c, c);
    for (int c = 0; c < nch; ++c) {
        // stage c has landed (for every wave after the barrier) and every
        // wave is done with the stage the next copy overwrites
        if (c + 1 < nch && (c + 1) % CPL != 0)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DQ_STAGE_VM) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        const int cn = c + DQ_NST - 1;           // within this piece of the key list only
        if (cn < nch && cn / CPL == c / CPL) stage(cn, cn % DQ_NST);
        const char* st = smem + (c % DQ_NST) * DQ_STAGE;
        const __bf16* dsT = reinterpret_cast<const __bf16*>(st);
        const char* kt = st + DQ_DS;
#pragma unroll
        for (int k4 = 0; k4 < 2; ++k4) {
            // A: dS[m = head][k = slot], slots 16 k4 + 4 g + s4 (+ 8); B: the K
            // rows of the same slots, column block db0 + b; B reads run up to
            // five blocks ahead of the products
            const int sr = 16 * k4 + 4 * g + s4;
            const int u = 8 * hb + 4 * hh + (t16 & 3);
            u32x2 a0, a1, bb[9][2];
            tr_read2o<0>(a0, a1, lds_addr(dsT + dsoff(sr, u)), lds_addr(dsT + dsoff(sr + 8, u)));
            auto issue_b = [&](int b) {
                const int col = 32 * (db0 + b) + 16 * hh + 4 * (t16 & 3);
                tr_read2o<0>(bb[b][0], bb[b][1], lds_addr(kt + loff<QROW>(sr, col)),
                             lds_addr(kt + loff<QROW>(sr + 8, col)));
            };
#pragma unroll
            for (int b = 0; b < 5; ++b) issue_b(b);
            static_for<0, 9>([&](auto bI) {
                constexpr int b = decltype(bI)::value;
                constexpr int after = (b + 4 < 8 ? b + 4 : 8) - b;   // B pairs issued after this one
                lgkm_wait<2 * after>(a0, a1, bb[b][0]);
                lgkm_wait<2 * after>(bb[b][1]);
                acc[b] = mfma32(cat_u(a0, a1), cat_u(bb[b][0], bb[b][1]), acc[b]);
                if constexpr (b + 5 < 9) issue_b(b + 5);
            });
        }
        if ((c + 1) % CPL == 0 && c + 1 < nch) {
            // the next piece of the key list, then the ring refilled from it
            __syncthreads();
            load_keys((c + 1) * DQ_CH);
            __syncthreads();
            for (int cc = c + 1; cc < c + DQ_NST && cc < nch; ++cc) stage(cc, cc % DQ_NST);
        }
    }
    // dQ: C[m = head][n = column]
#pragma unroll
    for (int b = 0; b < 9; ++b) {
        const int col = 32 * (db0 + b) + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int h = hg * HG + hb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            dQ[((size_t)h * Nq + i) * DQK + col] = (__bf16)(acc[b][r] * scale);
        }
    }
}

// ----------------------------------------------------------------------------
// Transpose of the index lists (counting sort by key, stable in row order).
// hist: per block of RB rows, how many of its pairs name each key.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void sidx_hist_kernel(const int* __restrict__ idx,
                                                        const int* __restrict__ tlen,
                                                        int* __restrict__ cnt, int Nq, int Nkv,
                                                        int topk) {
    __shared__ int h[MAX_NKV];
    const int b = blockIdx.x;
    for (int j = threadIdx.x; j < Nkv; j += 256) h[j] = 0;
    __syncthreads();
    const int i1 = min(Nq, (b + 1) * RB);
    for (int i = b * RB; i < i1; ++i) {
        const int nval = valid_slots(tlen, i, topk);
        const int* irow = idx + (size_t)i * topk;
        for (int s = threadIdx.x; s < nval; s += 256) {
            const int key = slot_key(irow, s, nval, Nkv);
            if (key >= 0) atomicAdd(&h[key], 1);
        }
    }
    __syncthreads();
    for (int j = threadIdx.x; j < Nkv; j += 256) cnt[(size_t)b * Nkv + j] = h[j];
}

// Per key (one thread each): the exclusive running count over row blocks, in
// place, and the key's total into off[j].
__global__ __launch_bounds__(64) void sidx_colscan_kernel(int* __restrict__ cnt, int* __restrict__ off,
                                                          int nb, int Nkv) {
    const int j = blockIdx.x * 64 + threadIdx.x;
    if (j >= Nkv) return;
    int run = 0;
    int b = 0;
    for (; b + 8 <= nb; b += 8) {                 // eight independent loads in flight
        int c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = cnt[(size_t)(b + u) * Nkv + j];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            cnt[(size_t)(b + u) * Nkv + j] = run;
            run += c[u];
        }
    }
    for (; b < nb; ++b) {
        const int c = cnt[(size_t)b * Nkv + j];
        cnt[(size_t)b * Nkv + j] = run;
        run += c;
    }
    off[j] = run;
}

// One workgroup: exclusive scan of the per-key totals into off[0..Nkv].
__global__ __launch_bounds__(1024) void sidx_keyscan_kernel(int* __restrict__ off, int Nkv) {
    __shared__ int part[1024];
    const int t = threadIdx.x;
    const int per = (Nkv + 1023) / 1024;
    const int j0 = t * per, j1 = min(Nkv, j0 + per);
    int run_total = 0;
    for (int j = j0; j < j1; ++j) run_total += off[j];
    part[t] = run_total;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {          // inclusive scan of the partials
        const int v = t >= d ? part[t - d] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    int base = t ? part[t - 1] : 0;
    for (int j = j0; j < j1; ++j) {
        const int tot = off[j];
        off[j] = base;
        base += tot;
    }
    if (t == 1023) off[Nkv] = part[1023];
}

// Fill: rows of a block in order, the slots of one row in parallel; a key
// appears at most once per row in well-formed lists (duplicates within a row
// are still placed, in an unspecified order between themselves).
__global__ __launch_bounds__(256) void sidx_fill_kernel(const int* __restrict__ idx,
                                                        const int* __restrict__ tlen,
                                                        const int* __restrict__ cnt,
                                                        const int* __restrict__ off,
                                                        int* __restrict__ list, int Nq, int Nkv,
                                                        int topk) {
    __shared__ int h[MAX_NKV];
    const int b = blockIdx.x;
    for (int j = threadIdx.x; j < Nkv; j += 256) h[j] = 0;
    __syncthreads();
    const int i1 = min(Nq, (b + 1) * RB);
    for (int i = b * RB; i < i1; ++i) {
        const int nval = valid_slots(tlen, i, topk);
        const int* irow = idx + (size_t)i * topk;
        for (int s = threadIdx.x; s < nval; s += 256) {
            const int key = slot_key(irow, s, nval, Nkv);
            if (key >= 0) {
                const int r = atomicAdd(&h[key], 1);
                list[off[key] + cnt[(size_t)b * Nkv + key] + r] = i * topk + s;
            }
        }
        __syncthreads();
    }
}

// Per key: dV_j = sum over its (row, slot) pairs and head groups of the stored
// contributions, dK_j = scale * the same sum of the dK parts.  One workgroup
// of RW waves per key: the key's list (in its fixed order) is cut into RW
// contiguous segments, wave w sums segment w in list order, and the segment
// sums are added in segment order, so that the result does not depend on
// timing.  (A key can collect thousands of rows, the first keys of a causal
// selection most of all; one wave per key left those few keys to set the
// kernel's length.)  A contribution row is 2176 bytes of fp16: lane l takes
// the 16-byte chunks l (dV columns 8l ..) and 64 + l (dK columns 8l ..) and
// the value 1024 + l (dK column 512 + l), multiplies them by the row's
// power-of-two scales (exact) and adds in fp32; rows are loaded four at a
// time so that 12 loads per lane are in flight.
constexpr int RW = 4;                            // waves per key

__global__ __launch_bounds__(RW * 64) void sbwd_reduce_kernel(const _Float16* __restrict__ part,
                                                             const float2* __restrict__ pscale,
                                                             const int* __restrict__ off,
                                                             const int* __restrict__ list,
                                                             __bf16* __restrict__ dK,
                                                             __bf16* __restrict__ dV, int Nkv, int G,
                                                             int topk, float scale) {
    static_assert(PW == 2 * 512 + 64, "row layout: two 1 KiB chunks per 64 lanes and 64 values");
    typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
    typedef float f32x8 __attribute__((ext_vector_type(8)));
    __shared__ f32x8 red8[RW - 1][2][64];
    __shared__ float redt[RW - 1][64];
    const int lane = threadIdx.x & 63;
    const int w = wave_id();
    const int j = blockIdx.x;
    f32x8 av = {}, ak = {};
    float at = 0.f;
    // contribution rows of key j: (list entry e, head group hg), e in list order
    const int e0 = off[j];
    const int nrows = (off[j + 1] - e0) * G;
    auto row_of = [&](int r) -> size_t {
        const int pr = list[e0 + r / G];          // i * topk + s
        const int i = pr / topk, s = pr - i * topk;
        return ((size_t)i * G + r % G) * topk + s;
    };
    auto add_row = [&](f16x8 v, f16x8 k, _Float16 t, float2 m) {
        av += __builtin_convertvector(v, f32x8) * m.x;
        ak += __builtin_convertvector(k, f32x8) * m.y;
        at += (float)t * m.y;
    };
    // this wave's segment [r0, r1)
    const int r0 = (int)((long long)nrows * w / RW), r1 = (int)((long long)nrows * (w + 1) / RW);
    int r = r0;
    for (; r + 4 <= r1; r += 4) {
        f16x8 v[4], k[4];
        _Float16 t[4];
        float2 m[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const size_t pr = row_of(r + u);
            const _Float16* row = part + pr * PW;
            // non-temporal: every contribution is read once (1.7% faster)
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const f16x8*>(row) + lane);
            k[u] = __builtin_nontemporal_load(reinterpret_cast<const f16x8*>(row) + 64 + lane);
            t[u] = __builtin_nontemporal_load(row + 1024 + lane);
            m[u] = pscale[pr];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) add_row(v[u], k[u], t[u], m[u]);
    }
    for (; r < r1; ++r) {
        const size_t pr = row_of(r);
        const _Float16* row = part + pr * PW;
        add_row(__builtin_nontemporal_load(reinterpret_cast<const f16x8*>(row) + lane),
                __builtin_nontemporal_load(reinterpret_cast<const f16x8*>(row) + 64 + lane),
                __builtin_nontemporal_load(row + 1024 + lane), pscale[pr]);
    }
    // segment sums 1 .. RW-1 to wave 0, added in segment order
    if (w > 0) {
        red8[w - 1][0][lane] = av;
        red8[w - 1][1][lane] = ak;
        redt[w - 1][lane] = at;
    }
    __syncthreads();
    if (w != 0) return;
#pragma unroll
    for (int q = 0; q < RW - 1; ++q) {
        av += red8[q][0][lane];
        ak += red8[q][1][lane];
        at += redt[q][lane];
    }
    typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
    *reinterpret_cast<bf16x8v*>(dV + (size_t)j * DV + 8 * lane) = __builtin_convertvector(av, bf16x8v);
    *reinterpret_cast<bf16x8v*>(dK + (size_t)j * DQK + 8 * lane) = __builtin_convertvector(ak * scale, bf16x8v);
    dK[(size_t)j * DQK + 512 + lane] = (__bf16)(at * scale);
}

}  // namespace sp

// ----------------------------------------------------------------------------
// Host launchers
// ----------------------------------------------------------------------------
static int sp_tpad(int topk) { return ((topk + sp::SBW_CHUNK - 1) / sp::SBW_CHUNK) * sp::SBW_CHUNK; }

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace: [block counts nb x Nkv int32][off Nkv + 1 int32][pair list
// Nq x topk int32][dS^T Nq x G x tpad x 64 bf16][contribution scales Nq x G x
// topk float2][contributions Nq x G x topk x 1088 fp16], each segment
// 256-byte aligned.  Nothing needs initialising: every word read is written
// earlier in the same call.
size_t sparse_bwd_workspace_bytes(int Hq, int Nq, int Nkv, int topk) {
    const size_t G = (size_t)Hq / sp::HG;
    const size_t nb = ((size_t)Nq + sp::RB - 1) / sp::RB;
    return al256(nb * Nkv * 4) + al256(((size_t)Nkv + 1) * 4) + al256((size_t)Nq * topk * 4) +
           al256((size_t)Nq * G * sp_tpad(topk) * sp::HG * 2) + al256((size_t)Nq * G * topk * 8) +
           al256((size_t)Nq * G * topk * sp::PW * 2);
}

hipError_t launch_sparse_fwd(const void* q, const void* k, const void* v, const int* idx,
                             const int* tlen, void* o, float* lse, int Hq, int Nq, int Nkv,
                             int topk, float scale, hipStream_t stream) {
    const int G = Hq / sp::HG;
    if ((long long)Nq * G == 0) return hipSuccess;
    constexpr int smem = sp::FwdSmem::bytes;
    hipError_t e = hipFuncSetAttribute((const void*)sp::sfwd_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sp::sfwd_kernel, dim3(Nq * G), dim3(256), smem, stream, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, idx, tlen, (__bf16*)o, lse, Hq, Nq, Nkv,
                       topk, scale);
    return hipGetLastError();
}

hipError_t launch_sparse_bwd(const void* q, const void* k, const void* v, const void* dO,
                             const float* lse, const float* D, const int* idx, const int* tlen,
                             void* dq, void* dk, void* dv, void* workspace, int Hq, int Nq, int Nkv,
                             int topk, float scale, hipStream_t stream, hipEvent_t main_start,
                             hipEvent_t main_stop) {
    if (Nkv == 0 && Nq == 0) return hipSuccess;
    const int G = Hq / sp::HG;
    const int nb = (Nq + sp::RB - 1) / sp::RB;
    const int tpad = sp_tpad(topk);
    char* ws = (char*)workspace;
    int* cnt = (int*)ws;
    ws += al256((size_t)nb * Nkv * 4);
    int* off = (int*)ws;
    ws += al256(((size_t)Nkv + 1) * 4);
    int* list = (int*)ws;
    ws += al256((size_t)Nq * topk * 4);
    __bf16* dsw = (__bf16*)ws;
    ws += al256((size_t)Nq * G * tpad * sp::HG * 2);
    float2* pscale = (float2*)ws;
    ws += al256((size_t)Nq * G * topk * 8);
    _Float16* part = (_Float16*)ws;

    hipError_t e;
    if (nb > 0) {
        hipLaunchKernelGGL(sp::sidx_hist_kernel, dim3(nb), dim3(256), 0, stream, idx, tlen, cnt, Nq,
                           Nkv, topk);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (Nkv > 0) {
        hipLaunchKernelGGL(sp::sidx_colscan_kernel, dim3((Nkv + 63) / 64), dim3(64), 0, stream, cnt,
                           off, nb, Nkv);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(sp::sidx_keyscan_kernel, dim3(1), dim3(1024), 0, stream, off, Nkv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (nb > 0) {
        hipLaunchKernelGGL(sp::sidx_fill_kernel, dim3(nb), dim3(256), 0, stream, idx, tlen, cnt, off,
                           list, Nq, Nkv, topk);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((long long)Nq * G > 0) {
        constexpr int smem_main = sp::BwdSmem::bytes;
        constexpr int smem_dq = sp::DQ_SMEM;
        if ((e = hipFuncSetAttribute((const void*)sp::sbwd_main_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, smem_main)) != hipSuccess)
            return e;
        if ((e = hipFuncSetAttribute((const void*)sp::sbwd_dq_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, smem_dq)) != hipSuccess)
            return e;
        if (main_start && (e = hipEventRecord(main_start, stream)) != hipSuccess) return e;
        hipLaunchKernelGGL(sp::sbwd_main_kernel, dim3(Nq * G), dim3(sp::SBW_WAVES * 64), smem_main, stream,
                           (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)dO,
                           lse, D, idx, tlen, dsw, part, pscale, Hq, Nq, Nkv, topk, tpad, scale);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (main_stop && (e = hipEventRecord(main_stop, stream)) != hipSuccess) return e;
        hipLaunchKernelGGL(sp::sbwd_dq_kernel, dim3(Nq * G), dim3(256), smem_dq, stream,
                           (const __bf16*)k, dsw, idx, tlen, (__bf16*)dq, Hq, Nq, Nkv, topk, tpad,
                           scale);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (Nkv > 0) {
        hipLaunchKernelGGL(sp::sbwd_reduce_kernel, dim3(Nkv), dim3(sp::RW * 64), 0, stream, part,
                           pscale, off, list, (__bf16*)dk, (__bf16*)dv, Nkv, G, topk, scale);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace attn
