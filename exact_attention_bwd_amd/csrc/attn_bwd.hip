// Exact attention backward for gfx950: preprocess (D), the fused backward
// kernel (dK, dV and fp32 dQ partials), the dQ workspace fill and the dQ
// convert.
//
// The method is the tiled backward of "Writing Speed-of-Light Attention
// Backward Kernel for 5090 in CUDA" (hoanh.space): sections "Precomputing D",
// "Main backward kernel" and the tiled-backward pseudocode after
// "Mathematical Formulation".  One workgroup owns one key/value tile K_j, V_j
// of one (batch, head), keeps dK_j and dV_j in registers, walks the query
// tiles i (from the diagonal tile when causal), recomputes S_ij and P_ij from
// the saved log-sum-exp L, and adds its dQ_i partial into an fp32 workspace
// with atomics; a second kernel rounds that workspace to bf16.
//
// CDNA4 mapping (not the page's SM120 one):
//  * 256 threads = 4 wave64s; the workgroup owns B_c = 128 keys, each wave 32
//    of them, so every wave's dK/dV rows are private to it (no reduction).
//  * S = Q K^T and dP = dO V^T use K and V as B operands held in VGPRs for the
//    whole workgroup; Q and dO rows come from LDS.  The accumulator layout of
//    S/dP puts one key per lane, which is exactly the A layout of P^T and
//    dS^T for dV = P^T dO and dK = dS^T Q, so P and dS never go through LDS for
//    those two products; the k index is relabelled consistently on the B side
//    (dO^T, Q^T kept in LDS in transposed, XOR-swizzled form).
//  * dQ = dS K needs dS with one query per lane, so dS goes through LDS once;
//    K^T for that product stays in VGPRs.
//  * The next Q/dO tile is fetched into registers while the current one is
//    computed, then written to LDS (row-major and transposed) between the two
//    workgroup barriers of an iteration.
//  * P = exp(scale * S - L) is evaluated as 2^(S * scale * log2 e - L * log2 e)
//    with v_exp_f32.
#include "common.hpp"
#include "launch.hpp"

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

// Zero an fp32 buffer of n4 float4 entries (the dQ workspace).
__global__ __launch_bounds__(256) void fill_zero_kernel(f32x4* __restrict__ p, long long n4) {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4;
         i += (long long)gridDim.x * 256)
        p[i] = z;
}

// dQ = bf16(scale * dQ_accum) for rows < N of every (batch, head).
template <int HD>
__global__ __launch_bounds__(256) void dq_convert_kernel(
    const float* __restrict__ acc, __bf16* __restrict__ dQ, int BH, int N, int n_pad,
    float scale) {
    constexpr int CPR = HD / 8;                 // 8-element chunks per row
    const long long total = (long long)BH * N * CPR;
    for (long long c = (long long)blockIdx.x * 256 + threadIdx.x; c < total;
         c += (long long)gridDim.x * 256) {
        const long long row = c / CPR;          // bh * N + n
        const int part = (int)(c % CPR);
        const long long bh = row / N;
        const long long n = row % N;
        const float* src = acc + ((size_t)(bh * n_pad + n) * HD + part * 8);
        const f32x4 a = *reinterpret_cast<const f32x4*>(src);
        const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
        f32x8 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = a[e] * scale;
            v[e + 4] = b[e] * scale;
        }
        *reinterpret_cast<bf16x8*>(dQ + (size_t)row * HD + part * 8) = to_bf16x8(v);
    }
}

// ----------------------------------------------------------------------------
// Fused backward main kernel
// ----------------------------------------------------------------------------
namespace bwd {

constexpr int BC = 128;          // keys per workgroup (4 waves x 32)
constexpr int BR = 64;           // query rows per iteration (2 blocks of 32)
constexpr int NT = 256;          // threads

// Row-major tiles in LDS are padded by 16 bytes per row so that the 16-byte
// operand reads of eight consecutive rows fall on distinct banks.
template <int HD> struct Smem {
    static constexpr int QS = HD + 8;            // Q / dO row stride (elements)
    static constexpr int SS = BC + 8;            // dS row stride
    static constexpr int KTS = BC + 8;           // K^T staging row stride
    // transposed Q^T / dO^T: HD rows of BR = 64 queries = 16 chunks of 8 bytes,
    // unpadded, chunk index XOR-swizzled by the row.
    static constexpr int TS = BR;
    static constexpr int off_q = 0;
    static constexpr int off_do = off_q + BR * QS * 2;
    static constexpr int off_qt = off_do + BR * QS * 2;
    static constexpr int off_dot = off_qt + HD * TS * 2;
    static constexpr int off_ds = off_dot + HD * TS * 2;
    static constexpr int off_l = off_ds + BR * SS * 2;
    static constexpr int off_d = off_l + BR * 4;
    static constexpr int bytes = off_d + BR * 4;
    // K^T staging (prologue only) overlays the Q and dO tiles.
    static constexpr int off_kt = 0;
    static_assert(HD * KTS * 2 <= off_qt, "K^T staging must fit in the Q/dO area");
};

// Swizzled position (in elements) of 8-byte chunk `ch` (0..15) of row `r` of a
// transposed tile with 64 elements per row.  The XOR keeps both the operand
// reads (16 consecutive rows, same chunk) and the staging writes (rows 8
// apart, same chunk) on distinct banks.
__device__ __forceinline__ int tswz(int r, int ch) {
    return r * BR + (((ch ^ (r ^ (r >> 4))) & 15) << 2);
}

// Per-thread share of one Q (or dO) tile: 4 consecutive rows x 8 columns.
template <int HD> struct TileRegs {
    u32x4 q[4], g[4];
    float l, d;
};

template <int HD>
__device__ __forceinline__ void load_tile(TileRegs<HD>& tr, const __bf16* Qh, const __bf16* dOh,
                                          const float* Lh, const float* Dh, int q0, int N) {
    constexpr int CG = HD / 8;                   // column groups
    const int t = threadIdx.x;
    if (t < 16 * CG) {
        const int cg = t % CG, rg = t / CG;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = q0 + rg * 4 + r;
            if (row < N) {
                tr.q[r] = gload16(Qh + (size_t)row * HD + cg * 8);
                tr.g[r] = gload16(dOh + (size_t)row * HD + cg * 8);
            } else {
                tr.q[r] = u32x4{0u, 0u, 0u, 0u};
                tr.g[r] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
    if (t < BR) {
        const int row = q0 + t;
        // rows past the end get L = +inf, so P = 2^-inf = 0 there
        tr.l = row < N ? Lh[row] * kLog2e : __builtin_inff();
        tr.d = row < N ? Dh[row] : 0.f;
    }
}

template <int HD>
__device__ __forceinline__ void store_tile(const TileRegs<HD>& tr, char* smem) {
    using S = Smem<HD>;
    constexpr int CG = HD / 8;
    const int t = threadIdx.x;
    __bf16* Qs = reinterpret_cast<__bf16*>(smem + S::off_q);
    __bf16* dOs = reinterpret_cast<__bf16*>(smem + S::off_do);
    __bf16* QT = reinterpret_cast<__bf16*>(smem + S::off_qt);
    __bf16* dOT = reinterpret_cast<__bf16*>(smem + S::off_dot);
    if (t < 16 * CG) {
        const int cg = t % CG, rg = t / CG;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            *reinterpret_cast<u32x4*>(Qs + (rg * 4 + r) * S::QS + cg * 8) = tr.q[r];
            *reinterpret_cast<u32x4*>(dOs + (rg * 4 + r) * S::QS + cg * 8) = tr.g[r];
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int drow = cg * 8 + c;
            *reinterpret_cast<u32x2*>(QT + tswz(drow, rg)) =
                column4(tr.q[0], tr.q[1], tr.q[2], tr.q[3], c);
            *reinterpret_cast<u32x2*>(dOT + tswz(drow, rg)) =
                column4(tr.g[0], tr.g[1], tr.g[2], tr.g[3], c);
        }
    }
    if (t < BR) {
        reinterpret_cast<float*>(smem + S::off_l)[t] = tr.l;
        reinterpret_cast<float*>(smem + S::off_d)[t] = tr.d;
    }
}

template <int HD, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1)))
void bwd_main_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                     const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                     const float* __restrict__ Lse, const float* __restrict__ Dd,
                     float* __restrict__ dQacc, __bf16* __restrict__ dK,
                     __bf16* __restrict__ dV, int BH, int N, int n_pad, float scale) {
    using S = Smem<HD>;
    constexpr int KSD = HD / 16;                 // k steps over the head dim
    constexpr int DB = HD / 32;                  // 32-wide blocks of the head dim
    constexpr int DQT = 2 * DB / 4;              // dQ output tiles per wave
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int l32 = lane & 31;
    const int g = lane >> 5;

    const int tc = (N + BC - 1) / BC;
    const int logical = xcd_remap(blockIdx.x, BH * tc);
    const int bh = logical / tc;
    const int j = logical % tc;                  // heavy (small j) first when causal
    const int k0 = j * BC;

    const size_t head = (size_t)bh * N * HD;
    const __bf16* Qh = Q + head;
    const __bf16* Kh = K + head;
    const __bf16* Vh = V + head;
    const __bf16* dOh = dO + head;
    const float* Lh = Lse + (size_t)bh * N;
    const float* Dh = Dd + (size_t)bh * N;
    float* dQh = dQacc + (size_t)bh * n_pad * HD;

    // ---- K, V as B operands of S = Q K^T and dP = dO V^T (this wave's 32 keys)
    bf16x8 kb[KSD], vb[KSD];
    {
        const int key = k0 + w * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            if (key < N) {
                kb[ks] = __builtin_bit_cast(bf16x8, gload16(Kh + (size_t)key * HD + ks * 16 + g * 8));
                vb[ks] = __builtin_bit_cast(bf16x8, gload16(Vh + (size_t)key * HD + ks * 16 + g * 8));
            } else {
                kb[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
                vb[ks] = kb[ks];
            }
        }
    }

    // ---- K^T as the B operand of dQ = dS K: staged transposed through LDS once
    const int dq_db = (DB == 4) ? w : (w & 1);   // this wave's 32 head-dim columns of dQ
    const int dq_qb0 = (DB == 4) ? 0 : (w >> 1); // first query block it covers
    bf16x8 kt[BC / 16];
    {
        __bf16* KT = reinterpret_cast<__bf16*>(smem + S::off_kt);
        constexpr int CG = HD / 8;
        for (int blk = threadIdx.x; blk < (BC / 4) * CG; blk += NT) {
            const int cg = blk % CG, rg = blk / CG;
            u32x4 r4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = k0 + rg * 4 + r;
                r4[r] = key < N ? gload16(Kh + (size_t)key * HD + cg * 8) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int c = 0; c < 8; ++c)
                *reinterpret_cast<u32x2*>(KT + (cg * 8 + c) * S::KTS + rg * 4) =
                    column4(r4[0], r4[1], r4[2], r4[3], c);
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < BC / 16; ++ks)
            kt[ks] = lds_read16(KT + (dq_db * 32 + l32) * S::KTS + ks * 16 + g * 8);
        __syncthreads();
    }

    f32x16 dv[DB], dk[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) {
        dv[b] = zero16();
        dk[b] = zero16();
    }

    const int tr_count = (N + BR - 1) / BR;
    const int it0 = CAUSAL ? (k0 / BR) : 0;

    const __bf16* Qs = reinterpret_cast<const __bf16*>(smem + S::off_q);
    const __bf16* dOs = reinterpret_cast<const __bf16*>(smem + S::off_do);
    const __bf16* QT = reinterpret_cast<const __bf16*>(smem + S::off_qt);
    const __bf16* dOT = reinterpret_cast<const __bf16*>(smem + S::off_dot);
    __bf16* dSs = reinterpret_cast<__bf16*>(smem + S::off_ds);
    const float* Ls = reinterpret_cast<const float*>(smem + S::off_l);
    const float* Ds = reinterpret_cast<const float*>(smem + S::off_d);

    TileRegs<HD> pre;
    load_tile<HD>(pre, Qh, dOh, Lh, Dh, it0 * BR, N);
    store_tile<HD>(pre, smem);
    __syncthreads();

    const float sl2 = scale * kLog2e;
    const int key_lane = k0 + w * 32 + l32;      // this lane's key (accumulator column)

    for (int it = it0; it < tr_count; ++it) {
        const int q0 = it * BR;
        const bool has_next = it + 1 < tr_count;
        if (has_next) load_tile<HD>(pre, Qh, dOh, Lh, Dh, q0 + BR, N);

        // ---- S = Q K^T and dP = dO V^T for 64 queries x this wave's 32 keys
        f32x16 s[2], dp[2];
        s[0] = zero16(); s[1] = zero16(); dp[0] = zero16(); dp[1] = zero16();
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const bf16x8 a = lds_read16(Qs + (qb * 32 + l32) * S::QS + ks * 16 + g * 8);
                const bf16x8 b = lds_read16(dOs + (qb * 32 + l32) * S::QS + ks * 16 + g * 8);
                s[qb] = mfma32(a, kb[ks], s[qb]);
                dp[qb] = mfma32(b, vb[ks], dp[qb]);
            }
        }

        // ---- P = exp(scale*S - L), dS = P o (dP - D); masked entries give 0
        const bool need_mask = (k0 + BC > N) || (CAUSAL && (k0 + BC - 1 > q0));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int qrow = qb * 32 + rr * 8 + g * 4;          // 4 consecutive rows
                const f32x4 lv = *reinterpret_cast<const f32x4*>(Ls + qrow);
                const f32x4 dd = *reinterpret_cast<const f32x4*>(Ds + qrow);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = rr * 4 + e;
                    float x = s[qb][r] * sl2 - lv[e];
                    if (need_mask) {
                        const int qg = q0 + qrow + e;
                        const bool masked = (key_lane >= N) || (CAUSAL && key_lane > qg);
                        x = masked ? -__builtin_inff() : x;
                    }
                    const float p = __builtin_amdgcn_exp2f(x);
                    s[qb][r] = p;
                    dp[qb][r] = p * (dp[qb][r] - dd[e]);
                }
            }
        }

        // ---- P^T and dS^T as A operands (k = query, relabelled per lane group)
        bf16x8 pa[4], dsa[4];
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
            pa[k4] = pack_c8(s[k4 >> 1], (k4 & 1) * 8);
            dsa[k4] = pack_c8(dp[k4 >> 1], (k4 & 1) * 8);
        }

        // ---- dS to LDS, one query per row, for dQ = dS K
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int r = (k4 & 1) * 8 + e;
                const int qrow = (k4 >> 1) * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
                dSs[qrow * S::SS + w * 32 + l32] = dsa[k4][e];
            }
        }

        // ---- dV += P^T dO, dK += dS^T Q (B operands from the transposed tiles)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int drow = db * 32 + l32;
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) {
                const bf16x8 bo = cat44(lds_read8(dOT + tswz(drow, 4 * k4 + g)),
                                        lds_read8(dOT + tswz(drow, 4 * k4 + 2 + g)));
                const bf16x8 bq = cat44(lds_read8(QT + tswz(drow, 4 * k4 + g)),
                                        lds_read8(QT + tswz(drow, 4 * k4 + 2 + g)));
                dv[db] = mfma32(pa[k4], bo, dv[db]);
                dk[db] = mfma32(dsa[k4], bq, dk[db]);
            }
        }

        __syncthreads();                        // dS complete; Q/dO tiles free
        if (has_next) store_tile<HD>(pre, smem);

        // ---- dQ_i partial = dS K over this workgroup's 128 keys, added atomically
#pragma unroll
        for (int tq = 0; tq < DQT; ++tq) {
            const int qb = dq_qb0 + tq;
            f32x16 acc = zero16();
#pragma unroll
            for (int ks = 0; ks < BC / 16; ++ks) {
                const bf16x8 a = lds_read16(dSs + (qb * 32 + l32) * S::SS + ks * 16 + g * 8);
                acc = mfma32(a, kt[ks], acc);
            }
            float* dst = dQh + (size_t)(q0 + qb * 32) * HD + dq_db * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = (r >> 2) * 8 + g * 4 + (r & 3);
                unsafeAtomicAdd(dst + (size_t)row * HD, acc[r]);
            }
        }
        __syncthreads();                        // next tile visible; dS reads done
    }

    // ---- epilogue: dK = scale * sum dS^T Q, dV = sum P^T dO, bf16 (RNE) stores
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + w * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
            if (key < N) {
                const size_t off = head + (size_t)key * HD + db * 32 + l32;
                dK[off] = (__bf16)(dk[db][r] * scale);
                dV[off] = (__bf16)dv[db][r];
            }
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
    if (d == 128) {
        hipLaunchKernelGGL(bwd_preprocess_kernel<128>, dim3(grid_for(rows, 16, 8192)), dim3(256), 0,
                           stream, (const __bf16*)o, (const __bf16*)dO, D, rows);
    } else {
        hipLaunchKernelGGL(bwd_preprocess_kernel<64>, dim3(grid_for(rows, 32, 8192)), dim3(256), 0,
                           stream, (const __bf16*)o, (const __bf16*)dO, D, rows);
    }
    return hipGetLastError();
}

size_t bwd_workspace_bytes(int BH, int N, int d) {
    const size_t n_pad = (size_t)((N + bwd::BR - 1) / bwd::BR) * bwd::BR;
    return (size_t)BH * n_pad * d * sizeof(float);
}

template <int HD, bool CAUSAL>
static hipError_t launch_main(const void* q, const void* k, const void* v, const void* dO,
                              const float* lse, const float* D, float* acc, void* dk, void* dv,
                              int BH, int N, int n_pad, float scale, hipStream_t stream) {
    using S = bwd::Smem<HD>;
    auto kern = bwd::bwd_main_kernel<HD, CAUSAL>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, S::bytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int tc = (N + bwd::BC - 1) / bwd::BC;
    hipLaunchKernelGGL(kern, dim3(BH * tc), dim3(bwd::NT), S::bytes, stream, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, (const __bf16*)dO, lse, D, acc,
                       (__bf16*)dk, (__bf16*)dv, BH, N, n_pad, scale);
    return hipGetLastError();
}

hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                      const float* D, void* dq, void* dk, void* dv, void* workspace, int BH, int N,
                      int d, bool causal, float scale, hipStream_t stream, hipEvent_t main_start,
                      hipEvent_t main_stop) {
    if ((long long)BH * N == 0) return hipSuccess;
    const int n_pad = ((N + bwd::BR - 1) / bwd::BR) * bwd::BR;
    float* acc = (float*)workspace;
    const long long n4 = (long long)BH * n_pad * d / 4;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n4, 256 * 4, 4096)), dim3(256), 0, stream,
                       (f32x4*)acc, n4);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (main_start && (e = hipEventRecord(main_start, stream)) != hipSuccess) return e;
    if (d == 128) {
        e = causal ? launch_main<128, true>(q, k, v, dO, lse, D, acc, dk, dv, BH, N, n_pad, scale, stream)
                   : launch_main<128, false>(q, k, v, dO, lse, D, acc, dk, dv, BH, N, n_pad, scale, stream);
    } else {
        e = causal ? launch_main<64, true>(q, k, v, dO, lse, D, acc, dk, dv, BH, N, n_pad, scale, stream)
                   : launch_main<64, false>(q, k, v, dO, lse, D, acc, dk, dv, BH, N, n_pad, scale, stream);
    }
    if (e != hipSuccess) return e;
    if (main_stop && (e = hipEventRecord(main_stop, stream)) != hipSuccess) return e;
    const long long chunks = (long long)BH * N * (d / 8);
    if (d == 128) {
        hipLaunchKernelGGL(dq_convert_kernel<128>, dim3(grid_for(chunks, 256 * 4, 8192)), dim3(256), 0,
                           stream, acc, (__bf16*)dq, BH, N, n_pad, scale);
    } else {
        hipLaunchKernelGGL(dq_convert_kernel<64>, dim3(grid_for(chunks, 256 * 4, 8192)), dim3(256), 0,
                           stream, acc, (__bf16*)dq, BH, N, n_pad, scale);
    }
    return hipGetLastError();
}

}  // namespace attn
