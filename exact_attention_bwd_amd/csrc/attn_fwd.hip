// Exact attention forward for gfx950: tiled online softmax producing O and the
// natural-log row log-sum-exp L that the backward consumes.
//
// The method is the FlashAttention-2 forward described in the
// s-samchenko/flash_attention_cuda README (online softmax with running max m,
// normaliser l and rescale by exp(m_old - m_new); one workgroup per query tile
// of one (batch, head); normalisation deferred to the end) and in the B200
// attention blog (iaroslavelistratov.github.io), Chapter 1 "Work
// Parallelization" and Chapter 8 (exponentials evaluated in base 2 with log2 e
// folded into the softmax scale).  L_i = log sum_j exp(S_ij) follows
// "Mathematical Formulation" of the attention-backward page.
//
// CDNA4 mapping:
//  * 256 threads = 4 wave64s, 128 query rows per workgroup, 32 per wave.
//  * Each wave computes S^T = K Q^T: K rows (A operand) come from LDS, this
//    wave's Q rows (B operand) stay in VGPRs for the whole loop.  In the
//    accumulator layout every lane then owns one query row, so the running
//    max / sum are per-lane values combined with a single exchange between
//    the two 32-lane halves, and the O rescale is one multiply per register.
//  * O^T = V^T P^T: P^T (B operand) comes straight from the S^T accumulators;
//    V^T (A operand) is staged transposed and XOR-swizzled in LDS.
//  * The next K/V tile is fetched into registers during the current one.
#include <type_traits>

#include "asm_ops.hpp"
#include "common.hpp"
#include "fwd_sched.hpp"
#include "launch.hpp"
#include "tiles.hpp"


namespace attn {
namespace fwd {

constexpr int BM = 128;          // query rows per workgroup
constexpr int BN = 64;           // keys per iteration
constexpr int NT = 256;

template <int HD> struct Smem {
    static constexpr int KS = HD + 8;            // K row stride (elements), padded
    static constexpr int off_k = 0;
    static constexpr int off_vt = off_k + BN * KS * 2;
    static constexpr int bytes = off_vt + HD * BN * 2;
};

// Swizzled element offset of 8-byte chunk `ch` (0..15) of row `r` of the
// transposed V tile (64 keys per row).
__device__ __forceinline__ int tswz(int r, int ch) {
    return r * BN + (((ch ^ (r ^ (r >> 4))) & 15) << 2);
}

template <int HD> struct KVRegs {
    u32x4 k[4], v[4];
};

template <int HD>
__device__ __forceinline__ void load_kv(KVRegs<HD>& kr, const __bf16* Kh, const __bf16* Vh, int n0,
                                        int N) {
    constexpr int CG = HD / 8;
    const int t = threadIdx.x;
    if (t < (BN / 4) * CG) {
        const int cg = t % CG, rg = t / CG;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = n0 + rg * 4 + r;
            if (key < N) {
                kr.k[r] = gload16(Kh + (size_t)key * HD + cg * 8);
                kr.v[r] = gload16(Vh + (size_t)key * HD + cg * 8);
            } else {
                kr.k[r] = u32x4{0u, 0u, 0u, 0u};
                kr.v[r] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
}

template <int HD>
__device__ __forceinline__ void store_kv(const KVRegs<HD>& kr, char* smem) {
    using S = Smem<HD>;
    constexpr int CG = HD / 8;
    const int t = threadIdx.x;
    __bf16* Ks = reinterpret_cast<__bf16*>(smem + S::off_k);
    __bf16* VT = reinterpret_cast<__bf16*>(smem + S::off_vt);
    if (t < (BN / 4) * CG) {
        const int cg = t % CG, rg = t / CG;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            *reinterpret_cast<u32x4*>(Ks + (rg * 4 + r) * S::KS + cg * 8) = kr.k[r];
#pragma unroll
        for (int c = 0; c < 8; ++c)
            *reinterpret_cast<u32x2*>(VT + tswz(cg * 8 + c, rg)) =
                column4(kr.v[0], kr.v[1], kr.v[2], kr.v[3], c);
    }
}

template <int HD, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                const __bf16* __restrict__ V, __bf16* __restrict__ O, float* __restrict__ Lse,
                int BH, int H, int G, int N, float scale) {
    using S = Smem<HD>;
    constexpr int KSD = HD / 16;
    constexpr int DB = HD / 32;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int lane = threadIdx.x & 63;
    const int w = wave_id();
    const int l32 = lane & 31;
    const int g = lane >> 5;

    const int tq = (N + BM - 1) / BM;
    const int logical = xcd_remap(blockIdx.x, BH * tq);
    const int bh = logical / tq;
    // causal: the last query tiles see the most keys, so they go first
    const int qt = CAUSAL ? (tq - 1 - logical % tq) : (logical % tq);
    const int q0 = qt * BM;

    const size_t head = (size_t)bh * N * HD;
    const __bf16* Qh = Q + head;
    // grouped-query attention: query head h of a batch reads K / V head h / G
    const size_t kvhead = (size_t)kv_head(bh, H, G) * N * HD;
    const __bf16* Kh = K + kvhead;
    const __bf16* Vh = V + kvhead;

    // this lane's query row (the accumulator column of S^T and O^T)
    const int qrow = q0 + w * 32 + l32;
    bf16x8 qb[KSD];
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks)
        qb[ks] = qrow < N ? __builtin_bit_cast(bf16x8, gload16(Qh + (size_t)qrow * HD + ks * 16 + g * 8))
                          : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});

    f32x16 o[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) o[b] = zero16();
    float m = -__builtin_inff();                 // running max, log2 units
    float l = 0.f;                               // this lane's share of the normaliser

    const int tk = (N + BN - 1) / BN;
    int kt_end = tk;
    if (CAUSAL) {
        const int last_q = min(q0 + BM, N) - 1;
        kt_end = min(tk, last_q / BN + 1);
    }

    const __bf16* Ks = reinterpret_cast<const __bf16*>(smem + S::off_k);
    const __bf16* VT = reinterpret_cast<const __bf16*>(smem + S::off_vt);
    const float sl2 = scale * kLog2e;

    KVRegs<HD> pre;
    load_kv<HD>(pre, Kh, Vh, 0, N);
    store_kv<HD>(pre, smem);
    __syncthreads();

    for (int kt = 0; kt < kt_end; ++kt) {
        const int n0 = kt * BN;
        const bool has_next = kt + 1 < kt_end;
        if (has_next) load_kv<HD>(pre, Kh, Vh, n0 + BN, N);

        // ---- S^T = K Q^T: 64 keys x this wave's 32 queries
        f32x16 s[2];
        s[0] = zero16();
        s[1] = zero16();
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8 a = lds_read16(Ks + (kb * 32 + l32) * S::KS + ks * 16 + g * 8);
                s[kb] = mfma32(a, qb[ks], s[kb]);
            }
        }

        // ---- scale, mask, running max
        const bool need_mask = (n0 + BN > N) || (CAUSAL && (n0 + BN - 1 > q0));
        float mt = -__builtin_inff();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = s[kb][r] * sl2;
                if (need_mask) {
                    const int key = n0 + kb * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
                    const bool masked = (key >= N) || (CAUSAL && key > qrow);
                    x = masked ? -__builtin_inff() : x;
                }
                s[kb][r] = x;
                mt = fmaxf(mt, x);
            }
        }
        mt = wave_max_pair32(mt);
        const float m_new = fmaxf(m, mt);
        // m_new is finite: every row sees key 0 in the first tile
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        m = m_new;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(s[kb][r] - m_new);
                s[kb][r] = p;
                rs += p;
            }
        }
        l = l * alpha + rs;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[b][r] *= alpha;

        // ---- O^T += V^T P^T
        bf16x8 pb[4];
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) pb[k4] = pack_c8(s[k4 >> 1], (k4 & 1) * 8);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int drow = db * 32 + l32;
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) {
                const bf16x8 a = cat44(lds_read8(VT + tswz(drow, 4 * k4 + g)),
                                       lds_read8(VT + tswz(drow, 4 * k4 + 2 + g)));
                o[db] = mfma32(a, pb[k4], o[db]);
            }
        }

        if (has_next) {
            __syncthreads();                    // everyone is done with K/V tile kt
            store_kv<HD>(pre, smem);
            __syncthreads();
        }
    }

    // ---- finalise: O = O / l, L = (m + log2 l) * ln 2
    const float lt = l + __shfl_xor(l, 32);
    const float inv = 1.f / lt;
    if (qrow < N) {
        __bf16* Oh = O + head + (size_t)qrow * HD;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                bf16x4 v4;
#pragma unroll
                for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(o[db][rr * 4 + e] * inv);
                *reinterpret_cast<bf16x4*>(Oh + db * 32 + rr * 8 + g * 4) = v4;
            }
        }
        if (g == 0) Lse[(size_t)bh * N + qrow] = (m + __builtin_amdgcn_logf(lt)) * kLn2;
    }
}


// ----------------------------------------------------------------------------
// d = 128: fwd_w64_kernel.  One workgroup of 4 wave64s (one per SIMD) per
// 256-row query tile; wave w owns rows 64 w .. + 63 as two 32-row blocks qb.
//
//  * Every K or V^T operand read from LDS feeds two MFMAs (one per row
//    block), which halves the LDS traffic per product against 32 rows per
//    wave.  Q (the B operand of S^T = K Q^T) stays in the AGPR file for the
//    whole loop, next to the O^T accumulators.
//  * K and V tiles of 64 keys arrive by direct buffer -> LDS copies into a
//    ring of 2 K slots and 3 V slots; one barrier per tile orders the copies
//    against the reads (see the slot rules at the loop).
//  * Software pipeline over key tiles t: iteration t runs the S phase (the
//    32 MFMAs of S(t+1) = K_{t+1} Q^T, with the exponentials of tile t's
//    second key block on the VALU) and then the PV phase (the 32 MFMAs of
//    O^T += V_t^T P_t^T, with the row max of S(t+1) and the exponentials of
//    its first key block on the VALU).  Each MFMA slot ends in a
//    sched_barrier that keeps the compiler from regrouping the work.
//  * Online softmax with a lazy rescale (B200 attention blog, Chapter 8,
//    conditional rescaling): the exponent offset m of a row only moves when
//    the running max exceeds it by more than 8 (log2 units), so
//    P = 2^(S scale log2 e - m) <= 256 and O and l are rescaled by
//    2^(m_old - m_new) only then (a wave-uniform branch, taken only by waves
//    with such a row).
//  * Every LDS read is issued from assembly at a fixed point and waited for
//    with the count FwdSched derives from the issue order.
// ----------------------------------------------------------------------------
constexpr int WBM = 256;                 // query rows per workgroup

struct WSmem {
    static constexpr int TILE = BN * 128 * 2;        // one K or V tile: 16 KiB
    static constexpr int off_k = 0;                  // K slots 0, 1
    static constexpr int off_v = 2 * TILE;           // V slots 0, 1, 2
    static constexpr int bytes = 5 * TILE;
};

// S^T products: result in VGPRs (the VALU reads it); the K and Q operands
// come from AGPRs
__device__ __forceinline__ void mfma_q(f32x16& c, const bf16x8& a, const bf16x8& b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "a"(a), "a"(b));
}

__device__ __forceinline__ void mfma_q0(f32x16& c, const bf16x8& a, const bf16x8& b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(c) : "a"(a), "a"(b));
}

// O^T accumulation: V^T and P^T operands from VGPRs, result in AGPRs
__device__ __forceinline__ void mfma_o(f32x16& c, const bf16x8& a, const bf16x8& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// c += a0 b0 + a1 b1 with operands just written by the VALU: the wait states
// before cover the VALU write -> MFMA operand read, those after keep the
// compiler's next writes of these registers clear of the MFMAs' operand reads
// (the compiler does not see MFMAs issued from assembly).
__device__ __forceinline__ void mfma_mask(f32x16& c, const bf16x8& a0, const bf16x8& a1, const bf16x8& b0,
                                          const bf16x8& b1) {
    asm volatile(
        "s_nop 4\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %3, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0\n\t"
        "s_nop 7"
        : "+v"(c)
        : "v"(a0), "v"(a1), "v"(b0), "v"(b1));
}

// max(a, b, c) without the canonicalising v_max the compiler puts in front of
// every fmaxf operand that it cannot prove canonical (the MFMA results)
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// x of lane l combined with x of lane l ^ 32: v_permlane32_swap exchanges the
// upper half of one register with the lower half of another, so both halves
// of a copy end up holding the other lane's value (no LDS involved)
__device__ __forceinline__ float pair_max(float x) {
    float y;
    asm volatile(
        "v_mov_b32 %1, %0\n\t"
        "s_nop 1\n\t"
        "v_permlane32_swap_b32 %0, %1\n\t"
        "s_nop 1\n\t"
        "v_max_f32 %0, %0, %1"
        : "+v"(x), "=&v"(y));
    return x;
}

__device__ __forceinline__ float pair_sum(float x) {
    float y;
    asm volatile(
        "v_mov_b32 %1, %0\n\t"
        "s_nop 1\n\t"
        "v_permlane32_swap_b32 %0, %1\n\t"
        "s_nop 1\n\t"
        "v_add_f32 %0, %0, %1"
        : "+v"(x), "=&v"(y));
    return x;
}

// first element of tile t + 1 whose exponential slot m of the PV phase
// evaluates (RB 32-row blocks per wave: slots 4 RB .. 16 RB - 1 take the
// 16 RB elements of key block 0)
constexpr int pv_e(int m, int RB) { return m <= 4 * RB ? 0 : ((m - 4 * RB) * 4) / 3; }

// 16 wait states tied to the accumulators a VALU instruction reads next
template <int RB>
__device__ __forceinline__ void settle(f32x16 (&s)[RB][2], int kb) {
    if constexpr (RB == 2) asm volatile("s_nop 15" : "+v"(s[0][kb]), "+v"(s[1][kb]));
    else asm volatile("s_nop 15" : "+v"(s[0][kb]));
}

template <int RB>
__device__ __forceinline__ void settle_o(f32x16 (&o)[RB][4]) {
    if constexpr (RB == 2)
        asm volatile("s_nop 15\n\ts_nop 15"
                     : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]),
                       "+a"(o[1][0]), "+a"(o[1][1]), "+a"(o[1][2]), "+a"(o[1][3]));
    else
        asm volatile("s_nop 15\n\ts_nop 15" : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]));
}

// One work item of the d = 128 forward: query tile qt (256 rows) of flattened
// head bh.  RB = 2: 4 waves (one per SIMD), 64 rows each; RB = 1: 8 waves (two
// per SIMD), 32 rows each.  Both cover a 256-row query tile.  On return every
// wave has issued its last LDS read and its last copy has landed, but other
// waves may still read LDS: the caller passes a barrier before the next item.
template <bool CAUSAL, int RB>
__device__ __forceinline__ void fwd_w64_item(char* smem, const __bf16* __restrict__ Q,
                                             const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                                             __bf16* __restrict__ O, float* __restrict__ Lse, int H, int G,
                                             int N, float scale, int bh, int qt) {
    constexpr int HD = 128;
    constexpr int NW = 8 / RB;                   // waves per workgroup
    constexpr int EPT = 32 * RB;                 // softmax elements per lane per key tile
    constexpr int EH = EPT / 2;                  // of which key block 0
    constexpr int NS = 16 * RB;                  // MFMA slots per phase
    using SC = FwdSched;
    using S = WSmem;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    const int lane = threadIdx.x & 63;
    const int w = wave_id();
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int t16 = lane & 15;
    const int hh = (lane >> 4) & 1;
    const int s4 = t16 >> 2;

    const int q0 = qt * WBM;
    const int qrows = min(N - q0, WBM);
    const int qw = 32 * RB * w;                  // this wave's first row in the tile
    const size_t head = (size_t)bh * N * HD;
    // grouped-query attention: query head h of a batch reads K / V head h / G
    const size_t kvhead = (size_t)kv_head(bh, H, G) * N * HD;
    const __bf16* Kh = K + kvhead;
    const __bf16* Vh = V + kvhead;
    const int T = CAUSAL ? (q0 + qrows - 1) / BN + 1 : (N + BN - 1) / BN;   // key tiles

    // Q rows of this lane as B operands of S^T: Q[qw + 32 qb + l32][16 ks + 8 g ..]
    bf16x8 qa[RB][8];
    {
        const __amdgpu_buffer_rsrc_t qr = make_rsrc(Q + head + (size_t)q0 * HD, qrows * HD * 2);
        static_for<0, RB>([&](auto qbI) __attribute__((always_inline)) {
            constexpr int qb = decltype(qbI)::value;
            static_for<0, 8>([&](auto ksI) __attribute__((always_inline)) {
                constexpr int ks = decltype(ksI)::value;
                qa[qb][ks] = __builtin_bit_cast(
                    bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, ((qw + 32 * qb + l32) * HD + 8 * g) * 2,
                                                                  ks * 32, 0));
            });
        });
    }

    int voff[BN * (HD / 8) / 64 / NW];
    stage_offsets<HD, BN, NW>(voff, w, lane);
    // tiles at or past T (padding of the last iteration) are filled with zeros
    auto dma = [&](const __bf16* base, int tile, int lds_off) __attribute__((always_inline)) {
        const int n0 = tile * BN;
        const int bytes = tile < T ? min(N - n0, BN) * HD * 2 : 0;
        stage_rows_b<HD, BN, NW>(make_rsrc(base + (size_t)min(n0, N - 1) * HD, bytes), voff, smem + lds_off, w);
    };

    // row reads of K: chunk 2 ks + g of row 32 kb + l32 at (aK ^ 32 ks) + 8 KiB kb
    const uint32_t aK = lds_addr(smem) + (uint32_t)(roff<HD>(l32, g) * 2);
    uint32_t aKs[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) aKs[ks] = aK ^ (uint32_t)(ks * 32);
    // transposing reads of V (A operand V^T): rows 4 g + s4 (+ 16 k4, + 8),
    // columns 16 hh + 4 (t16 & 3) (+ 32 db); bases of the current V slot
    const int otr = roff4<HD>(g * 4 + s4, hh * 16 + 4 * (t16 & 3));
    uint32_t trv[4][2];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        trv[db][0] = lds_addr(smem + S::off_v) + (uint32_t)((otr ^ (db << 5)) * 2);
        trv[db][1] = lds_addr(smem + S::off_v) + (uint32_t)((((otr + 8 * HD) ^ (db << 5)) ^ 16) * 2);
    }

    f32x16 sa[RB][2], sb[RB][2];                 // S^T of tiles t (t even: sa) and t + 1
    f32x16 o[RB][4];                             // O^T, rows = head dim, in AGPRs
#pragma unroll
    for (int qb = 0; qb < RB; ++qb)
#pragma unroll
        for (int db = 0; db < 4; ++db) o[qb][db] = zero16();
    u32x4 pk[RB][4];                             // P^T operands (bf16 pairs)
    bf16x8 kop[16];
    u32x2 vop[16][2];
    float mrow[RB], lrow[RB], oa[RB], pmax[RB];
    bool pend[RB];
#pragma unroll
    for (int qb = 0; qb < RB; ++qb) {
        mrow[qb] = -__builtin_inff();            // exponent offset (log2 units)
        lrow[qb] = 0.f;                          // this lane's share of the normaliser
        oa[qb] = 1.f;                            // pending O rescale factor
        pend[qb] = false;
    }
    const float sl2 = scale * kLog2e;

    // operand j of an iteration whose K rows are in K slot KS
    auto issue = [&](auto jI, auto ksI) __attribute__((always_inline)) {
        constexpr int j = decltype(jI)::value, KS = decltype(ksI)::value;
        if constexpr (j < 16) {
            lds_ld_a<S::off_k + KS * S::TILE + (j >> 3) * 8192>(kop[j], aKs[j & 7]);
        } else {
            constexpr int v = j - 16;
            tr_read2o<(v >> 2) * 4096>(vop[v][0], vop[v][1], trv[v & 3][0], trv[v & 3][1]);
        }
    };
    // element e (0 .. EPT - 1) of a tile's S^T: p = 2^(S scale log2 e - m),
    // added to l and packed in pairs into the P^T operands.  e -> pair u = e / 2
    // of operand (row block qb, key step k4), k4 = u / (4 RB), qb = (u / 4) % RB,
    // dword i = u % 4, i.e. accumulator entry r = 8 (k4 % 2) + 2 i + e % 2 of
    // key block k4 / 2.  The first half of the elements is key block 0.
    struct Ix {
        int qb, kb, k4, i, r;
    };
    constexpr auto ix = [](int e) constexpr {
        const int u = e >> 1, k4 = u / (4 * RB);
        return Ix{(u >> 2) % RB, k4 >> 1, k4, u & 3, 8 * (k4 & 1) + 2 * (u & 3) + (e & 1)};
    };
    float phold = 0.f;                           // first element of a pair
    auto elem = [&](f32x16(&s)[RB][2], auto eI) __attribute__((always_inline)) {
        constexpr int e = decltype(eI)::value;
        constexpr Ix x = ix(e);
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[x.qb][x.kb][x.r], sl2, -mrow[x.qb]));
        lrow[x.qb] += p;
        if constexpr ((e & 1) == 0) {
            phold = p;
        } else {
            typedef float f32x2 __attribute__((ext_vector_type(2)));
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            pk[x.qb][x.k4][x.i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{phold, p}, bf16x2));
        }
    };
    // The same in two halves for the pipelined loop, issued one MFMA slot
    // apart so that no instruction waits for the exponential's result:
    // elem_exp leaves p in pbuf[e % 4], elem_sum adds it to l and packs pairs.
    float pbuf[4];
    auto elem_exp = [&](f32x16(&s)[RB][2], auto eI) __attribute__((always_inline)) {
        constexpr int e = decltype(eI)::value;
        constexpr Ix x = ix(e);
        pbuf[e & 3] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[x.qb][x.kb][x.r], sl2, -mrow[x.qb]));
    };
    auto elem_sum = [&](auto eI) __attribute__((always_inline)) {
        constexpr int e = decltype(eI)::value;
        constexpr Ix x = ix(e);
        lrow[x.qb] += pbuf[e & 3];
        // pinned here: the compiler would otherwise sink the sums and packs
        // towards their uses in the next iteration, past the rescale branch
        asm volatile("" : "+v"(lrow[x.qb]));
        if constexpr (e & 1) {
            typedef float f32x2 __attribute__((ext_vector_type(2)));
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            pk[x.qb][x.k4][x.i] = __builtin_bit_cast(
                uint32_t, __builtin_convertvector(f32x2{pbuf[(e - 1) & 3], pbuf[e & 3]}, bf16x2));
            asm volatile("" : "+v"(pk[x.qb][x.k4]));
        }
    };
    // Masking on the matrix core.  In block (qb, kb) of a tile, S^T entry
    // (key k, row q) must become -inf when k > thr(q) = min(row, N - 1) - key
    // offset.  With c(q) = clamp(thr(q) + 1, 0, 32), the product of the
    // constant 32 x 32 matrix [k >= k'] and the matrix B[k'][q] = -2^120 for
    // k' = c(q), else 0, adds -2^120 exactly to the masked entries and 0 to
    // the others; -2^120 scale log2 e underflows 2^x to 0 and never wins a
    // row max.  Only blocks that reach past a row or past N take it (a
    // wave-uniform branch around two MFMAs that update the block in place).
    // ALWAYS: no branch (the product adds zeros where nothing is masked);
    // used once, where a branch would only make the compiler copy the block
    auto mask = [&](f32x16(&s)[RB][2], auto qbI, auto kbI, int tile, auto alwaysI) __attribute__((always_inline)) {
        constexpr int qb = decltype(qbI)::value, kb = decltype(kbI)::value;
        const int kofs = tile * BN + 32 * kb;
        const int qrow0 = q0 + qw + 32 * qb;
        if (decltype(alwaysI)::value || (CAUSAL && kofs + 31 > qrow0) || kofs + 31 > N - 1) {
            const int lim = CAUSAL ? min(qrow0 + l32, N - 1) : N - 1;
            const int c = min(max(lim - kofs + 1, 0), 32);
            u32x4 bm[2];
            bf16x8 tri[2];                       // A operand: ones where key l32 >= k, k = 16 h + 8 g + e
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int idx = c - 16 * h - 8 * g;    // element of this lane's operand that is hit
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    bm[h][d] = (idx >> 1) == d ? ((idx & 1) ? 0xFB800000u : 0x0000FB80u) : 0u;
#pragma unroll
                for (int e = 0; e < 8; ++e) tri[h][e] = l32 >= 16 * h + 8 * g + e ? (__bf16)1.f : (__bf16)0.f;
            }
            mfma_mask(s[qb][kb], tri[0], tri[1], __builtin_bit_cast(bf16x8, bm[0]), __builtin_bit_cast(bf16x8, bm[1]));
        }
    };
    auto max8 = [&](float m, const f32x16& s, int h) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 8; r += 2) m = max3f(m, s[8 * h + r], s[8 * h + r + 1]);
        return m;
    };
    // new offset of row block qb from its tile max pmax (this lane's keys)
    auto combine = [&](int qb) __attribute__((always_inline)) {
        const float mx = pair_max(pmax[qb]);
        const float mn = __builtin_fmaxf(mrow[qb], mx * sl2);
        const bool need = mn > mrow[qb] + 8.f;
        const float alpha = __builtin_amdgcn_exp2f(mrow[qb] - mn);
        mrow[qb] = need ? mn : mrow[qb];
        lrow[qb] = need ? lrow[qb] * alpha : lrow[qb];
        oa[qb] = need ? alpha : 1.f;
        pend[qb] = __builtin_amdgcn_ballot_w64(need) != 0;
    };

    // ---- prologue: K_0, K_1, V_0; S(0); the first key block of tile 0
    dma(Kh, 0, S::off_k);
    dma(Kh, 1, S::off_k + S::TILE);
    dma(Vh, 0, S::off_v);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    static_for<0, SC::D>([&](auto jI) __attribute__((always_inline)) { issue(jI, I0{}); });
    static_for<0, NS>([&](auto mI) __attribute__((always_inline)) {
        constexpr int m = decltype(mI)::value, n = m / RB, qb = m % RB, kb = n >> 3, ks = n & 7;
        if constexpr (qb == 0) {
            if constexpr (SC::issues(SC::PRO, n)) issue(std::integral_constant<int, n + SC::D>{}, I0{});
            lgkm_wait_a<SC::wait(SC::PRO, n)>(kop[n]);
        }
        if constexpr (ks == 0) mfma_q0(sa[qb][kb], kop[n], qa[qb][ks]);
        else mfma_q(sa[qb][kb], kop[n], qa[qb][ks]);
        __builtin_amdgcn_sched_barrier(0);
    });
    // every wave has read K_0: its slot takes K_2; V_1 goes to V slot 1
    asm volatile("s_barrier" ::: "memory");
    dma(Kh, 2, S::off_k);
    dma(Vh, 1, S::off_v + S::TILE);
    static_for<0, SC::D>([&](auto jI) __attribute__((always_inline)) { issue(jI, I1{}); });   // K_1, iteration 0
    static_for<0, RB>([&](auto qbI) __attribute__((always_inline)) {
        mask(sa, qbI, I0{}, 0, std::true_type{});
        mask(sa, qbI, I1{}, 0, std::true_type{});
    });
    settle<RB>(sa, 0);
    settle<RB>(sa, 1);
#pragma unroll
    for (int qb = 0; qb < RB; ++qb) {
        pmax[qb] = max8(max8(max8(max8(-__builtin_inff(), sa[qb][0], 0), sa[qb][0], 1), sa[qb][1], 0), sa[qb][1], 1);
        combine(qb);
    }
    static_for<0, EH>([&](auto eI) __attribute__((always_inline)) { elem(sa, eI); });

    // ---- main loop.  Slot rules (B_t = the barrier of iteration t):
    //  * iteration t reads K_{t+1} (S phase; its first D operands are issued
    //    after B_{t-1}) and V_t (from the S phase's need point 16 - D on);
    //  * after B_t the wave copies K_{t+3} into the slot of K_{t+1} and
    //    V_{t+2} into the slot of V_{t-1}; every wave finished those reads
    //    before B_t, and each copy is complete (vmcnt(0)) and visible at
    //    B_{t+1}, before its first read.
    // The loop runs an even number of iterations; a padding tile T (zeros,
    // every key masked) contributes nothing.
    int vsl = 0;                                 // V slot of tile t: t % 3
    auto iter = [&](auto pI, int t) __attribute__((always_inline)) {
        constexpr int p = decltype(pI)::value;
        constexpr int KS = p ^ 1;               // K slot of tile t + 1
        f32x16(&sc)[RB][2] = p ? sb : sa;        // tile t
        f32x16(&sn)[RB][2] = p ? sa : sb;        // tile t + 1
        // ---- S phase: S(t+1); exponentials of tile t, key block 1
        static_for<0, NS>([&](auto mI) __attribute__((always_inline)) {
            constexpr int m = decltype(mI)::value, n = m / RB, qb = m % RB, kb = n >> 3, ks = n & 7;
            if constexpr (qb == 0) {
                if constexpr (SC::issues(SC::ITER, n))
                    issue(std::integral_constant<int, n + SC::D>{}, std::integral_constant<int, KS>{});
                lgkm_wait_a<SC::wait(SC::ITER, n)>(kop[n]);
            }
            if constexpr (ks == 0) mfma_q0(sn[qb][kb], kop[n], qa[qb][ks]);
            else mfma_q(sn[qb][kb], kop[n], qa[qb][ks]);
            elem_exp(sc, std::integral_constant<int, EH + m>{});
            if constexpr (m > 0) elem_sum(std::integral_constant<int, EH + m - 1>{});
            // mask and row max of S(t+1), key block 0 (its last products: the
            // slots before 8 RB)
            if constexpr (m == 8 * RB) {
                static_for<0, RB>([&](auto qbI) __attribute__((always_inline)) { mask(sn, qbI, I0{}, t + 1, std::false_type{}); });
                settle<RB>(sn, 0);
            }
            if constexpr (m > 8 * RB && m <= 12 * RB) {
                constexpr int b = (m - 8 * RB - 1) >> 2, h = (m - 8 * RB - 1) & 3;
                if constexpr (h == 0) pmax[b] = -__builtin_inff();
                pmax[b] = max3f(max3f(pmax[b], sn[b][0][4 * h], sn[b][0][4 * h + 1]), sn[b][0][4 * h + 2], sn[b][0][4 * h + 3]);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        // ---- PV phase: O^T += V_t^T P_t^T; row max and key block 0 of tile t + 1
        static_for<0, NS>([&](auto mI) __attribute__((always_inline)) {
            constexpr int m = decltype(mI)::value, v = m / RB, qb = m % RB, db = v & 3, k4 = v >> 2;
            constexpr int n = 16 + v;
            if constexpr (qb == 0) {
                if constexpr (n == SC::BARRIER_N) {
                    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
                    dma(Kh, t + 3, S::off_k + KS * S::TILE);
                    dma(Vh, t + 2, S::off_v + (vsl == 0 ? 2 : vsl - 1) * S::TILE);
                }
                if constexpr (SC::issues(SC::ITER, n))
                    issue(std::integral_constant<int, (n + SC::D) % SC::NOPS>{}, std::integral_constant<int, p>{});
                lgkm_wait<SC::wait(SC::ITER, n)>(vop[v][0], vop[v][1]);
            }
            mfma_o(o[qb][db], cat_u(vop[v][0], vop[v][1]), __builtin_bit_cast(bf16x8, pk[qb][k4]));
            if constexpr (m == 0) {
                static_for<0, RB>([&](auto qbI) __attribute__((always_inline)) { mask(sn, qbI, I1{}, t + 1, std::false_type{}); });
                settle<RB>(sn, 1);                // last S(t+1) products: the last S slots
                elem_sum(std::integral_constant<int, EPT - 1>{});   // tile t's last
            }
            if constexpr (m < 2 * RB) pmax[m >> 1] = max8(pmax[m >> 1], sn[m >> 1][1], m & 1);
            if constexpr (m >= 2 * RB && m < 3 * RB) combine(m - 2 * RB);
            if constexpr (m >= 4 * RB) {
                static_for<pv_e(m, RB), pv_e(m + 1, RB)>([&](auto eI) __attribute__((always_inline)) { elem_exp(sn, eI); });
            }
            if constexpr (m > 4 * RB) {
                static_for<pv_e(m - 1, RB), pv_e(m, RB)>([&](auto eI) __attribute__((always_inline)) { elem_sum(eI); });
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        static_for<pv_e(NS - 1, RB), pv_e(NS, RB)>([&](auto eI) __attribute__((always_inline)) { elem_sum(eI); });
        // lazy rescale of O^T, after the last product that used the old offset
        bool any = false;
#pragma unroll
        for (int qb = 0; qb < RB; ++qb) any = any || pend[qb];
        if (__builtin_expect(any, 0)) {
            settle_o<RB>(o);
            static_for<0, RB>([&](auto qbI) __attribute__((always_inline)) {
                constexpr int qb = decltype(qbI)::value;
                if (pend[qb]) {
                    static_for<0, 4>([&](auto dbI) __attribute__((always_inline)) {
                        o[qb][decltype(dbI)::value] *= oa[qb];
                        __builtin_amdgcn_sched_barrier(0);
                    });
                }
            });
        }
        // V slot of tile t + 1
        const int dv = vsl == 2 ? -2 * S::TILE : S::TILE;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            trv[db][0] += dv;
            trv[db][1] += dv;
        }
        vsl = vsl == 2 ? 0 : vsl + 1;
    };
    int t = 0;
    do {                                         // T >= 1
        iter(I0{}, t);
        iter(I1{}, t + 1);
        t += 2;
    } while (t < T);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // copies issued for tiles past the end

    // ---- O = O^T / l, L = (m + log2 l) ln 2
    settle_o<RB>(o);
    const __amdgpu_buffer_rsrc_t orc = make_rsrc(O + head + (size_t)q0 * HD, qrows * HD * 2);
    static_for<0, RB>([&](auto qbI) __attribute__((always_inline)) {
        constexpr int qb = decltype(qbI)::value;
        const float lt = pair_sum(lrow[qb]);
        const float inv = 1.f / lt;
        const int row = qw + 32 * qb + l32;
        static_for<0, 4>([&](auto dbI) __attribute__((always_inline)) {
            constexpr int db = decltype(dbI)::value;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                bf16x4 v4;
#pragma unroll
                for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(o[qb][db][rr * 4 + e] * inv);
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v4), orc,
                                                      (row * HD + db * 32 + rr * 8 + g * 4) * 2, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        if (g == 0 && row < qrows) Lse[(size_t)bh * N + q0 + row] = (mrow[qb] + __builtin_amdgcn_logf(lt)) * kLn2;
    });
}

// Persistent (B200 attention blog, Chapter 14 "Persistent"): a fixed grid, a
// multiple of 8 workgroups dealt round-robin to the 8 XCDs, each workgroup
// walking a fixed list of items.  Work order.  Causal: query tile qt sees 4 (qt + 1) key
// tiles, so the last tiles go first.  Each XCD takes every eighth head and
// works through them two at a time, longest tiles first within each pair, so
// that the few heads in flight on an XCD keep their K / V in its L2: the
// XCD's items are numbered in that order, and round m of its workgroups takes
// items m G8 .. m G8 + G8 - 1 (G8 workgroups per XCD) in snake order, the
// k-th workgroup the k-th item in even rounds and the (G8 - 1 - k)-th in odd
// ones, so that the heavy and light tiles of the rounds even out over the
// workgroups.  Other causal head counts: longest tiles first over all heads.
// Non-causal: one item per workgroup, the tiles of one head on one XCD.
template <bool CAUSAL, int RB>
__global__ __attribute__((amdgpu_flat_work_group_size(512 / RB, 512 / RB), amdgpu_waves_per_eu(3 - RB, 3 - RB)))
void fwd_w64_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                    const __bf16* __restrict__ V, __bf16* __restrict__ O, float* __restrict__ Lse,
                    int BH, int H, int G, int N, float scale) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tq = (N + WBM - 1) / WBM;
    const int items = BH * tq, per_xcd = (items + 7) / 8;
    if constexpr (!CAUSAL) {
        // equal items: one per workgroup (a loop would only add registers)
        const int logical = xcd_remap(blockIdx.x, items);
        fwd_w64_item<CAUSAL, RB>(smem, Q, K, V, O, Lse, H, G, N, scale, logical / tq, logical % tq);
        return;
    }
    const int G8 = gridDim.x / 8, x = blockIdx.x % 8, k = blockIdx.x / 8;
    for (int m = 0; m * G8 < per_xcd; ++m) {
        const int local = m * G8 + ((m & 1) ? G8 - 1 - k : k);
        const int item = local * 8 + x;          // the item's XCD is x, as its workgroup's
        if (local >= per_xcd || item >= items) continue;
        int bh, qt;
        if (CAUSAL && BH % 16 == 0) {
            const int t = item / 8;
            const int grp = t / (2 * tq), r = t % (2 * tq);
            qt = tq - 1 - r / 2;
            bh = (2 * grp + (r & 1)) * 8 + x;
        } else {
            bh = item % BH;
            qt = tq - 1 - item / BH;
        }
        fwd_w64_item<CAUSAL, RB>(smem, Q, K, V, O, Lse, H, G, N, scale, bh, qt);
        __syncthreads();                         // every wave is done with the LDS slots
    }
}

}  // namespace fwd

template <int HD, bool CAUSAL>
static hipError_t launch_fwd_t(const void* q, const void* k, const void* v, void* o, float* lse,
                               int BH, int H, int G, int N, float scale, hipStream_t stream) {
    using S = fwd::Smem<HD>;
    auto kern = fwd::fwd_kernel<HD, CAUSAL>;
    const int tq = (N + fwd::BM - 1) / fwd::BM;
    hipLaunchKernelGGL(kern, dim3(BH * tq), dim3(fwd::NT), S::bytes, stream, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, BH, H, G, N, scale);
    return hipGetLastError();
}

template <bool CAUSAL>
static hipError_t launch_fwd_w64(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int BH, int H, int G, int N, float scale, hipStream_t stream) {
    using S = fwd::WSmem;
    constexpr int RB = 1;                        // 8 waves of 32 rows (RB = 2 ran slower: one wave's issue bound it)
    auto kern = fwd::fwd_w64_kernel<CAUSAL, RB>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, S::bytes);
    if (e != hipSuccess) return e;
    // causal: one workgroup per CU (LDS and registers allow no more), a
    // multiple of 8; non-causal: one per item
    const int tq = (N + fwd::WBM - 1) / fwd::WBM;
    int dev = 0, cus = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    const int grid = CAUSAL ? std::min((BH * tq + 7) / 8 * 8, std::max(8, cus / 8 * 8)) : BH * tq;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(512 / RB), S::bytes, stream, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, BH, H, G, N, scale);
    return hipGetLastError();
}

hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                      int H, int G, int N, int d, bool causal, float scale, hipStream_t stream) {
    if ((long long)BH * N == 0) return hipSuccess;
    if (d == 128)
        return causal ? launch_fwd_w64<true>(q, k, v, o, lse, BH, H, G, N, scale, stream)
                      : launch_fwd_w64<false>(q, k, v, o, lse, BH, H, G, N, scale, stream);
    return causal ? launch_fwd_t<64, true>(q, k, v, o, lse, BH, H, G, N, scale, stream)
                  : launch_fwd_t<64, false>(q, k, v, o, lse, BH, H, G, N, scale, stream);
}

}  // namespace attn
