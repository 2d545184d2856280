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
#include "common.hpp"
#include "launch.hpp"

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
                int BH, int N, float scale) {
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
    const __bf16* Kh = K + head;
    const __bf16* Vh = V + head;

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

}  // namespace fwd

template <int HD, bool CAUSAL>
static hipError_t launch_fwd_t(const void* q, const void* k, const void* v, void* o, float* lse,
                               int BH, int N, float scale, hipStream_t stream) {
    using S = fwd::Smem<HD>;
    auto kern = fwd::fwd_kernel<HD, CAUSAL>;
    const int tq = (N + fwd::BM - 1) / fwd::BM;
    hipLaunchKernelGGL(kern, dim3(BH * tq), dim3(fwd::NT), S::bytes, stream, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, BH, N, scale);
    return hipGetLastError();
}

hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                      int N, int d, bool causal, float scale, hipStream_t stream) {
    if ((long long)BH * N == 0) return hipSuccess;
    if (d == 128)
        return causal ? launch_fwd_t<128, true>(q, k, v, o, lse, BH, N, scale, stream)
                      : launch_fwd_t<128, false>(q, k, v, o, lse, BH, N, scale, stream);
    return causal ? launch_fwd_t<64, true>(q, k, v, o, lse, BH, N, scale, stream)
                  : launch_fwd_t<64, false>(q, k, v, o, lse, BH, N, scale, stream);
}

}  // namespace attn
