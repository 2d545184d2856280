/*
 * attn_mi355x.h -- C ABI of the exact-attention library for AMD MI355X (gfx950).
 *
 * Fused exact scaled-dot-product attention, FlashAttention-2 style: a forward
 * pass that emits O and the row log-sum-exp L, the backward preprocess
 * D = rowsum(dO o O), and the fused backward producing dQ, dK and dV.
 *
 * The operations are those of "Writing Speed-of-Light Attention Backward Kernel
 * for 5090 in CUDA" (hoanh.space), section "Mathematical Formulation":
 *     S  = scale * Q K^T + M            (M = 0, or -inf where key j > query i when causal)
 *     L_i = log sum_j exp(S_ij)          (natural log, of the scaled masked scores)
 *     P  = exp(S - L),  O = P V
 *     dV = P^T dO,  dP = dO V^T,  D = rowsum(dO o O),  dS = P o (dP - D 1^T)
 *     dQ = scale * dS K,  dK = scale * dS^T Q
 * The page writes scale = 1/sqrt(d); here it is an argument.
 *
 * Conventions shared by every entry point
 *  - Tensors are dense, row-major, [B, H, N, d] (d fastest), bf16 unless noted;
 *    L and D are fp32 [B, H, N].  Pointers are device pointers (memory from
 *    hipMalloc or a framework allocator on the current device).
 *  - bf16 pointers must be 16-byte aligned; fp32 pointers 4-byte aligned; the
 *    workspace 16-byte aligned.
 *  - d must be 64 or 128.  N >= 1 may be any length (a ragged last tile is
 *    masked).  B*H*N == 0 is a no-op that returns ATTN_OK.
 *  - The caller owns every buffer, including the workspace.  The library never
 *    allocates, frees or synchronises: all work is enqueued on `stream`
 *    (a hipStream_t; NULL = the default stream) and ATTN_OK means the launches
 *    were enqueued, not that they have finished.
 *  - Errors are returned, never thrown.  On a non-OK status nothing was
 *    enqueued (validation errors) or the HIP launch failed (ATTN_ERR_HIP);
 *    attn_last_error() returns a message for the calling thread.
 *  - Calls may run concurrently on different streams if their output and
 *    workspace buffers do not overlap.
 */
#ifndef ATTN_MI355X_H
#define ATTN_MI355X_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int attn_status;

#define ATTN_OK 0
#define ATTN_ERR_INVALID_ARG (-1)   /* null/misaligned pointer, negative size, non-finite scale */
#define ATTN_ERR_UNSUPPORTED (-2)   /* head dimension not in {64, 128}, sizes too large */
#define ATTN_ERR_HIP (-3)           /* a HIP launch or attribute call failed */
#define ATTN_ERR_WORKSPACE (-4)     /* workspace smaller than attn_bwd_workspace_bytes() */

/*
 * Forward pass (tiled online softmax; s-samchenko/flash_attention_cuda README,
 * FlashAttention-2 forward with running max m, normaliser l and rescale by
 * exp(m_old - m_new)).
 *   q, k, v : bf16 [B, H, N, d], read only
 *   o       : bf16 [B, H, N, d], written (O = P V, rounded to nearest even)
 *   lse     : fp32 [B, H, N], written: L_i, natural log of sum_j exp(S_ij)
 *   causal  : nonzero = key j visible to query i only if j <= i
 *   scale   : softmax scale applied to Q K^T (finite)
 */
attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int N, int d, int causal, float scale, void* stream);

/*
 * Backward preprocess (attention-backward page, section "Precomputing D"):
 *   D_i = sum_c dO_ic * O_ic, accumulated in fp32 from the bf16 inputs.
 *   o, dO : bf16 [B, H, N, d], read only;  D : fp32 [B, H, N], written.
 *   d may also be 512: the O and dO of the sparse path ([Hq, Nq, 512], i.e.
 *   B = 1, H = Hq, N = Nq) use this same entry point.
 */
attn_status attn_bwd_preprocess(const void* o, const void* dO, float* D, int B, int H, int N,
                                int d, void* stream);

/*
 * Size in bytes of a workspace that serves attn_bwd for both values of
 * `causal` (the larger of the two attn_bwd_workspace_bytes_ex sizes).  0 when
 * B*H*N == 0 or the shape is unsupported.
 */
size_t attn_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * Exact workspace size of attn_bwd / attn_bwd_gqa for this shape and masking
 * (Hkv = H for attn_bwd): on the causal d = 128 path, a control block of
 * 64 + B*H*ceil(N/256) ints (work-queue counters, status words, one progress
 * word per query head and 256-key tile); the row statistics L*log2(e) and D padded to the
 * 64-row query tile (2 x B*H*ceil(N/64)*64 fp32); one bf16 128 x 64 dS tile per
 * (batch*head, 64-row query tile i, 128-key tile j) -- for causal only the
 * tiles with j <= i/2, the lower triangle; a bf16 copy of K rearranged as
 * matrix-core operands (B*Hkv*ceil(N/128)*128*d*2 bytes; on the causal
 * d = 128 path one copy per query head, B*H*...); and, for grouped-query
 * shapes whose query heads are split over several workgroups (on the causal
 * d = 128 path: every query head its own part), fp32 partials of dK and dV
 * (2*parts*B*Hkv*N*d*4 bytes).  Each part is rounded up to 256 bytes.  0 when
 * B*H*N == 0 or the shape is unsupported.
 */
size_t attn_bwd_workspace_bytes_ex(int B, int H, int Hkv, int N, int d, int causal);

/*
 * Fused backward (attention-backward page: the tiled backward pseudocode and
 * section "Main backward kernel"): recomputes P = exp(scale*S - L) tile by tile
 * and forms dV = P^T dO, dP = dO V^T, dS = P o (dP - D), dQ = scale*dS K and
 * dK = scale*dS^T Q.  Work is split by 256-key (d = 128) or 128-key (d = 64)
 * tiles: each workgroup keeps its keys' dK and dV in registers over the query
 * tiles and stores every bf16 dS tile in `workspace`; dQ_i = scale *
 * sum_j dS_ij K_j is then reduced in fp32 registers, without atomics:
 *  - causal, d = 128: in the same, persistent kernel (about one workgroup per
 *    CU, each taking work items from its XCD's queue), by the item of the key
 *    tile on the diagonal of query tiles i, once the items of the earlier key
 *    tiles of that head have stored their dS tiles of those rows (their
 *    progress is published in the workspace);
 *  - otherwise: by a second, query-parallel kernel.
 * All launches are on `stream`.
 *   q, k, v, dO : bf16 [B, H, N, d], read only
 *   lse         : fp32 [B, H, N]  L from attn_fwd (natural log), read only
 *   D           : fp32 [B, H, N]  from attn_bwd_preprocess, read only
 *   dq, dk, dv  : bf16 [B, H, N, d], written
 *   workspace   : device scratch of at least attn_bwd_workspace_bytes(B,H,N,d)
 *                 bytes, or of attn_bwd_workspace_bytes_ex(B,H,H,N,d,causal) (its
 *                 content on entry is ignored and on exit unspecified; for the
 *                 causal d = 128 path its first 64 ints are the work queues'
 *                 counters and status words)
 *   causal, scale : as for attn_fwd (must match the forward that produced lse)
 * dQ, dK and dV are deterministic (bitwise reproducible for the same inputs).
 */
attn_status attn_bwd(const void* q, const void* k, const void* v, const void* dO,
                     const float* lse, const float* D, void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                     int causal, float scale, void* stream);

/*
 * Same as attn_bwd, for profiling: when main_start / main_stop (hipEvent_t
 * created by the caller) are non-NULL they are recorded on `stream`
 * immediately before and after the dominant kernel (the fused kernel, with
 * the one-workgroup sweep launched right after it, on the causal d = 128
 * path; the dK/dV kernel otherwise), so the caller can time it alone
 * (hipEventElapsedTime) without a profiler.
 */
attn_status attn_bwd_timed(const void* q, const void* k, const void* v, const void* dO,
                           const float* lse, const float* D, void* dq, void* dk, void* dv,
                           void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                           int causal, float scale, void* stream, void* main_start,
                           void* main_stop);

/*
 * ---------------------------------------------------------------------------
 * Grouped-query attention (GQA; MQA when Hkv = 1): Hkv key / value heads, each
 * shared by G = H / Hkv consecutive query heads, the dense counterpart of the
 * shared K/V head of the sparse path below (cudnn-frontend PR #684, DSA: all
 * query heads attend through one K/V head, and dK, dV are sums over heads).
 * Query head h of batch b reads K / V head h / G of batch b:
 *     S_h = scale * Q_h K_{h/G}^T + M,   O_h = softmax(S_h) V_{h/G}
 * and the backward forms dQ_h as for dense attention and
 *     dK_c = sum over the query heads h with h / G = c of scale * dS_h^T Q_h,
 *     dV_c = sum over the same heads of P_h^T dO_h.
 * Shapes: q, o, dO, dq  [B, H, N, d];  k, v, dk, dv  [B, Hkv, N, d];
 * lse, D fp32 [B, H, N].  Hkv must divide H (ATTN_ERR_INVALID_ARG otherwise);
 * everything else as for attn_fwd / attn_bwd, which are these calls with
 * Hkv = H.  The per-head sums of dK and dV are formed in fp32 in a fixed
 * order, in registers or as one partial per workgroup added by a reduction
 * kernel (causal d = 128: the fused kernel's items are the query heads, one
 * partial each); no atomics, so results are bitwise reproducible.
 */
attn_status attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                         int H, int Hkv, int N, int d, int causal, float scale, void* stream);

/* Workspace of attn_bwd_gqa that serves both values of `causal`:
 * max over causal of attn_bwd_workspace_bytes_ex(B, H, Hkv, N, d, causal).
 * 0 for invalid shapes. */
size_t attn_bwd_gqa_workspace_bytes(int B, int H, int Hkv, int N, int d);

/* Grouped-query backward: lse, D and dO per query head, dk / dv per K / V head. */
attn_status attn_bwd_gqa(const void* q, const void* k, const void* v, const void* dO,
                         const float* lse, const float* D, void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes, int B, int H, int Hkv, int N,
                         int d, int causal, float scale, void* stream);

/* attn_bwd_gqa with the dominant kernel bracketed by main_start / main_stop,
 * as attn_bwd_timed (the fused kernel and its sweep on the causal d = 128
 * path, the dK/dV kernel otherwise; the group reduction falls outside). */
attn_status attn_bwd_gqa_timed(const void* q, const void* k, const void* v, const void* dO,
                               const float* lse, const float* D, void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes, int B, int H, int Hkv, int N,
                               int d, int causal, float scale, void* stream, void* main_start,
                               void* main_stop);

/*
 * ---------------------------------------------------------------------------
 * Top-k sparse attention (cudnn-frontend PR #684, "Improve performance of
 * SM100 DSA backward kernel": DSA attention with one shared K/V head).
 * Query row i attends, for every head, to the keys its index list names:
 *     S_h,i,s = scale * Q[h,i] . K[idx[i,s]]   for the valid slots s of row i
 *     P = softmax over the valid slots,  O[h,i] = sum_s P_h,i,s V[idx[i,s]]
 * and the backward applies the dense formulas above to that gathered set, with
 *     dK[j] = scale * sum over (h, i, s : idx[i,s] = j) of dS_h,i,s Q[h,i]
 *     dV[j] =         sum over (h, i, s : idx[i,s] = j) of P_h,i,s dO[h,i].
 * Shapes (all dense, row-major, bf16 unless noted):
 *   q  [Hq, Nq, dqk]    k  [Nkv, dqk]    v  [Nkv, dv]
 *   o, dO  [Hq, Nq, dv]     lse, D  fp32 [Hq, Nq]
 *   idx    int32 [Nq, topk]: key indices of each row
 *   topk_len  int32 [Nq] or NULL: number of leading slots of each row in use
 *             (clamped to [0, topk]; NULL = all topk)
 * A slot is valid when it is in use and its index lies in [0, Nkv); other
 * slots (e.g. -1 padding) are ignored.  A row with no valid slot gets O = 0,
 * L = -inf and zero gradients.  Supported: dqk = 576, dv = 512, Hq a multiple
 * of 64 (heads are processed in groups of 64 that share each gathered K/V
 * row), Nkv <= 1048576 (backward: Nkv <= 16384, topk <= 65536).  Pointer
 * alignment as for the dense calls; idx and topk_len 4-byte aligned.
 */
attn_status attn_sparse_fwd(const void* q, const void* k, const void* v, const int* idx,
                            const int* topk_len, void* o, float* lse, int Hq, int Nq, int Nkv,
                            int dqk, int dv, int topk, float scale, void* stream);

/*
 * Workspace of attn_sparse_bwd: a per-row-block key histogram
 * (ceil(Nq/16) x Nkv int32), key offsets (Nkv + 1 int32), the transposed pair
 * list (Nq x topk int32), dS (Nq x Hq/64 x ceil(topk/256)*256 x 64 bf16), the
 * two power-of-two scales of each (row, head group, slot) (float2) and its
 * dK/dV contribution (Nq x Hq/64 x topk x 1088 fp16; 4.6 GB at Hq = 64,
 * Nq = 4096, topk = 512), each 256-byte aligned.  0 for unsupported or empty
 * problems.
 */
size_t attn_sparse_bwd_workspace_bytes(int Hq, int Nq, int Nkv, int dqk, int dv, int topk);

/*
 * Sparse backward.  lse from attn_sparse_fwd, D from attn_bwd_preprocess(o,
 * dO, D, 1, Hq, Nq, 512).  Writes dq [Hq, Nq, dqk], dk [Nkv, dqk], dv [Nkv, dv]
 * (every key row, zero for keys no row selected).  Kernels, all on `stream`:
 * a counting-sort transpose of the index lists (per key, its (row, slot)
 * pairs in row order), a per-row kernel that recomputes S, P, dP, dS for the
 * 64 heads of a group and stores dS and each slot's dK/dV contribution (fp16
 * times a power of two bounded from the slot's P, dS and the row's max |Q|,
 * |dO|, so a stored value carries a relative error of at most 2^-12), a
 * per-row dQ kernel, and a per-key fp32 reduction of the contributions in
 * that fixed order.  No floating-point atomics: results are reproducible,
 * except that a key repeated within one row's list is summed in an
 * unspecified order.
 */
attn_status attn_sparse_bwd(const void* q, const void* k, const void* v, const void* dO,
                            const float* lse, const float* D, const int* idx, const int* topk_len,
                            void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                            int Hq, int Nq, int Nkv, int dqk, int dv_dim, int topk, float scale,
                            void* stream);

/*
 * attn_sparse_bwd with caller-created hipEvent_t main_start / main_stop (may
 * be NULL) recorded on `stream` immediately before and after the per-row
 * backward kernel, for timing it alone.
 */
attn_status attn_sparse_bwd_timed(const void* q, const void* k, const void* v, const void* dO,
                                  const float* lse, const float* D, const int* idx,
                                  const int* topk_len, void* dq, void* dk, void* dv,
                                  void* workspace, size_t workspace_bytes, int Hq, int Nq, int Nkv,
                                  int dqk, int dv_dim, int topk, float scale, void* stream,
                                  void* main_start, void* main_stop);

/*
 * ---------------------------------------------------------------------------
 * Backward without allocation, for callers that cannot allocate device
 * memory (code under stream or graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): attn_bwd with its workspace in a static array of
 * attn_bwd_noalloc_max_workspace_bytes() bytes (64 MiB) that the library
 * holds on every device it runs on, until the process ends.  The array's
 * device address is looked up on the first call on a device (a set-up step
 * that allocates nothing); the call itself allocates and frees nothing.
 * Shapes whose attn_bwd_workspace_bytes_ex(B, H, H, N, d, causal) exceeds that
 * size are rejected with ATTN_ERR_WORKSPACE (e.g. causal d = 128 fits up to
 * about three heads of N = 4096).  Every call on one device uses the same
 * array: calls that overlap on a device (two streams, two threads) race and
 * give wrong results; serialise them.  Arguments, results and other errors
 * as attn_bwd.
 */
attn_status attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* dO,
                             const float* lse, const float* D, void* dq, void* dk, void* dv, int B,
                             int H, int N, int d, int causal, float scale, void* stream);

/* Size in bytes of attn_bwd_noalloc's static scratch (the largest workspace it serves). */
size_t attn_bwd_noalloc_max_workspace_bytes(void);

/* Message describing the last non-OK status returned on this thread ("" if none). */
const char* attn_last_error(void);

/* Library version string. */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_H */
