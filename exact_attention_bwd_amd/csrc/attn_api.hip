// C entry points of the attention library: argument validation, then the
// launchers.  No allocation, no synchronisation, no exceptions across the ABI.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/attn_mi355x.h"
#include "api_error.hpp"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

attn_status fail(attn_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

attn_status ok() {
    g_err[0] = '\0';
    return ATTN_OK;
}

attn_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Common shape checks.  Sets *empty when there is nothing to do.
attn_status check_shape(int B, int H, int N, int d, bool* empty) {
    if (B < 0 || H < 0 || N < 0) return fail(ATTN_ERR_INVALID_ARG, "negative size B=%d H=%d N=%d", B, H, N);
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dimension d=%d not in {64, 128}", d);
    const long long bh = (long long)B * H;
    *empty = (bh * N == 0);
    if (*empty) return ATTN_OK;
    // grid and index limits: B*H*ceil(N/64) workgroups, B*H*N rows, element offsets in 64 bits
    if (bh > (1LL << 24) || N > (1 << 26) || bh * (((long long)N + 63) / 64) > 0x7fffffffLL)
        return fail(ATTN_ERR_UNSUPPORTED, "sizes too large B*H=%lld N=%d", bh, N);
    return ATTN_OK;
}

// Grouped-query attention: Hkv key / value heads, each shared by H / Hkv query heads.
attn_status check_heads(int H, int Hkv) {
    if (Hkv < 1 || Hkv > H || H % Hkv != 0)
        return fail(ATTN_ERR_INVALID_ARG, "Hkv=%d does not divide H=%d", Hkv, H);
    return ATTN_OK;
}

attn_status check_ptr(const void* p, const char* name, uintptr_t align) {
    if (p == nullptr) return fail(ATTN_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned(p, align)) return fail(ATTN_ERR_INVALID_ARG, "%s is not %u-byte aligned", name, (unsigned)align);
    return ATTN_OK;
}

#define CHECK(expr)                         \
    do {                                    \
        attn_status _s = (expr);            \
        if (_s != ATTN_OK) return _s;       \
    } while (0)

}  // namespace

attn_status attn::report(attn_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

extern "C" {

attn_status attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                         int H, int Hkv, int N, int d, int causal, float scale, void* stream) {
    bool empty = false;
    CHECK(check_shape(B, H, N, d, &empty));
    if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale is not finite");
    if (empty) return ok();
    CHECK(check_heads(H, Hkv));
    CHECK(check_ptr(q, "q", 16));
    CHECK(check_ptr(k, "k", 16));
    CHECK(check_ptr(v, "v", 16));
    CHECK(check_ptr(o, "o", 16));
    CHECK(check_ptr(lse, "lse", 4));
    return hip_status(attn::launch_fwd(q, k, v, o, lse, B * H, H, H / Hkv, N, d, causal != 0, scale,
                                       (hipStream_t)stream),
                      "attn_fwd launch");
}

attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int N, int d, int causal, float scale, void* stream) {
    return attn_fwd_gqa(q, k, v, o, lse, B, H, H, N, d, causal, scale, stream);
}

attn_status attn_bwd_preprocess(const void* o, const void* dO, float* D, int B, int H, int N,
                                int d, void* stream) {
    bool empty = false;
    // the sparse path's O and dO are 512 wide
    CHECK(check_shape(B, H, N, d == 512 ? 128 : d, &empty));
    if (empty) return ok();
    CHECK(check_ptr(o, "o", 16));
    CHECK(check_ptr(dO, "dO", 16));
    CHECK(check_ptr(D, "D", 4));
    return hip_status(attn::launch_bwd_preprocess(o, dO, D, B * H, N, d, (hipStream_t)stream),
                      "attn_bwd_preprocess launch");
}

size_t attn_bwd_workspace_bytes_ex(int B, int H, int Hkv, int N, int d, int causal) {
    bool empty = false;
    if (check_shape(B, H, N, d, &empty) != ATTN_OK || empty) return 0;
    if (check_heads(H, Hkv) != ATTN_OK) return 0;
    return attn::bwd_workspace_bytes(B * H, H / Hkv, N, d, causal != 0);
}

size_t attn_bwd_gqa_workspace_bytes(int B, int H, int Hkv, int N, int d) {
    const size_t a = attn_bwd_workspace_bytes_ex(B, H, Hkv, N, d, 0);
    const size_t b = attn_bwd_workspace_bytes_ex(B, H, Hkv, N, d, 1);
    return a > b ? a : b;
}

size_t attn_bwd_workspace_bytes(int B, int H, int N, int d) {
    return attn_bwd_gqa_workspace_bytes(B, H, H, N, d);
}

attn_status attn_bwd_gqa_timed(const void* q, const void* k, const void* v, const void* dO,
                               const float* lse, const float* D, void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes, int B, int H, int Hkv, int N,
                               int d, int causal, float scale, void* stream, void* main_start,
                               void* main_stop) {
    bool empty = false;
    CHECK(check_shape(B, H, N, d, &empty));
    if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale is not finite");
    if (empty) return ok();
    CHECK(check_heads(H, Hkv));
    CHECK(check_ptr(q, "q", 16));
    CHECK(check_ptr(k, "k", 16));
    CHECK(check_ptr(v, "v", 16));
    CHECK(check_ptr(dO, "dO", 16));
    CHECK(check_ptr(lse, "lse", 4));
    CHECK(check_ptr(D, "D", 4));
    CHECK(check_ptr(dq, "dq", 16));
    CHECK(check_ptr(dk, "dk", 16));
    CHECK(check_ptr(dv, "dv", 16));
    CHECK(check_ptr(workspace, "workspace", 16));
    const size_t need = attn::bwd_workspace_bytes(B * H, H / Hkv, N, d, causal != 0);
    if (workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "workspace is %zu bytes, %zu needed", workspace_bytes, need);
    return hip_status(attn::launch_bwd(q, k, v, dO, lse, D, dq, dk, dv, workspace, B * H, H, H / Hkv,
                                       N, d, causal != 0, scale, (hipStream_t)stream,
                                       (hipEvent_t)main_start, (hipEvent_t)main_stop),
                      "attn_bwd launch");
}

attn_status attn_bwd_gqa(const void* q, const void* k, const void* v, const void* dO,
                         const float* lse, const float* D, void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes, int B, int H, int Hkv, int N,
                         int d, int causal, float scale, void* stream) {
    return attn_bwd_gqa_timed(q, k, v, dO, lse, D, dq, dk, dv, workspace, workspace_bytes, B, H, Hkv,
                              N, d, causal, scale, stream, nullptr, nullptr);
}

attn_status attn_bwd_timed(const void* q, const void* k, const void* v, const void* dO,
                           const float* lse, const float* D, void* dq, void* dk, void* dv,
                           void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                           int causal, float scale, void* stream, void* main_start, void* main_stop) {
    return attn_bwd_gqa_timed(q, k, v, dO, lse, D, dq, dk, dv, workspace, workspace_bytes, B, H, H, N,
                              d, causal, scale, stream, main_start, main_stop);
}

attn_status attn_bwd(const void* q, const void* k, const void* v, const void* dO,
                     const float* lse, const float* D, void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                     int causal, float scale, void* stream) {
    return attn_bwd_gqa_timed(q, k, v, dO, lse, D, dq, dk, dv, workspace, workspace_bytes, B, H, H, N,
                              d, causal, scale, stream, nullptr, nullptr);
}

// ---------------------------------------------------------------------------
// Top-k sparse attention
// ---------------------------------------------------------------------------
namespace {

attn_status check_sparse(int Hq, int Nq, int Nkv, int dqk, int dv, int topk, bool bwd) {
    if (Hq < 0 || Nq < 0 || Nkv < 0 || topk < 0)
        return fail(ATTN_ERR_INVALID_ARG, "negative size Hq=%d Nq=%d Nkv=%d topk=%d", Hq, Nq, Nkv, topk);
    if (dqk != 576 || dv != 512)
        return fail(ATTN_ERR_UNSUPPORTED, "sparse head dims (d_qk=%d, d_v=%d) are not (576, 512)", dqk, dv);
    if (Hq % 64 != 0) return fail(ATTN_ERR_UNSUPPORTED, "Hq=%d is not a multiple of 64", Hq);
    if (Nkv > (1 << 20)) return fail(ATTN_ERR_UNSUPPORTED, "Nkv=%d above 1048576", Nkv);
    if (bwd && Nkv > 16384) return fail(ATTN_ERR_UNSUPPORTED, "sparse backward: Nkv=%d above 16384", Nkv);
    if (bwd && topk > 65536) return fail(ATTN_ERR_UNSUPPORTED, "sparse backward: topk=%d above 65536", topk);
    if ((long long)Nq * topk > 0x7fffffffLL || (long long)Nq * (Hq / 64) > 0x7fffffffLL)
        return fail(ATTN_ERR_UNSUPPORTED, "sizes too large Nq=%d topk=%d Hq=%d", Nq, topk, Hq);
    return ATTN_OK;
}

}  // namespace

attn_status attn_sparse_fwd(const void* q, const void* k, const void* v, const int* idx,
                            const int* topk_len, void* o, float* lse, int Hq, int Nq, int Nkv,
                            int dqk, int dv, int topk, float scale, void* stream) {
    CHECK(check_sparse(Hq, Nq, Nkv, dqk, dv, topk, false));
    if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale is not finite");
    if ((long long)Hq * Nq == 0) return ok();
    CHECK(check_ptr(q, "q", 16));
    CHECK(check_ptr(o, "o", 16));
    CHECK(check_ptr(lse, "lse", 4));
    if (Nkv > 0) {
        CHECK(check_ptr(k, "k", 16));
        CHECK(check_ptr(v, "v", 16));
    }
    if (topk > 0) CHECK(check_ptr(idx, "idx", 4));
    if (topk_len) CHECK(check_ptr(topk_len, "topk_len", 4));
    return hip_status(attn::launch_sparse_fwd(q, k, v, idx, topk_len, o, lse, Hq, Nq, Nkv, topk,
                                              scale, (hipStream_t)stream),
                      "attn_sparse_fwd launch");
}

size_t attn_sparse_bwd_workspace_bytes(int Hq, int Nq, int Nkv, int dqk, int dv, int topk) {
    if (check_sparse(Hq, Nq, Nkv, dqk, dv, topk, true) != ATTN_OK) return 0;
    if ((long long)Hq * Nq == 0 && Nkv == 0) return 0;
    return attn::sparse_bwd_workspace_bytes(Hq, Nq, Nkv, topk);
}

attn_status attn_sparse_bwd_timed(const void* q, const void* k, const void* v, const void* dO,
                                  const float* lse, const float* D, const int* idx,
                                  const int* topk_len, void* dq, void* dk, void* dv,
                                  void* workspace, size_t workspace_bytes, int Hq, int Nq, int Nkv,
                                  int dqk, int dvd, int topk, float scale, void* stream,
                                  void* main_start, void* main_stop) {
    CHECK(check_sparse(Hq, Nq, Nkv, dqk, dvd, topk, true));
    if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale is not finite");
    const bool rows = (long long)Hq * Nq > 0;
    if (!rows && Nkv == 0) return ok();
    if (rows) {
        CHECK(check_ptr(q, "q", 16));
        CHECK(check_ptr(dO, "dO", 16));
        CHECK(check_ptr(lse, "lse", 4));
        CHECK(check_ptr(D, "D", 4));
        CHECK(check_ptr(dq, "dq", 16));
    }
    if (Nkv > 0) {
        CHECK(check_ptr(k, "k", 16));
        CHECK(check_ptr(v, "v", 16));
        CHECK(check_ptr(dk, "dk", 16));
        CHECK(check_ptr(dv, "dv", 16));
    }
    if ((long long)Nq * topk > 0) CHECK(check_ptr(idx, "idx", 4));
    if (topk_len) CHECK(check_ptr(topk_len, "topk_len", 4));
    CHECK(check_ptr(workspace, "workspace", 16));
    const size_t need = attn::sparse_bwd_workspace_bytes(Hq, Nq, Nkv, topk);
    if (workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "workspace is %zu bytes, %zu needed", workspace_bytes, need);
    return hip_status(attn::launch_sparse_bwd(q, k, v, dO, lse, D, idx, topk_len, dq, dk, dv,
                                              workspace, Hq, Nq, Nkv, topk, scale,
                                              (hipStream_t)stream, (hipEvent_t)main_start,
                                              (hipEvent_t)main_stop),
                      "attn_sparse_bwd launch");
}

attn_status attn_sparse_bwd(const void* q, const void* k, const void* v, const void* dO,
                            const float* lse, const float* D, const int* idx, const int* topk_len,
                            void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                            int Hq, int Nq, int Nkv, int dqk, int dvd, int topk, float scale,
                            void* stream) {
    return attn_sparse_bwd_timed(q, k, v, dO, lse, D, idx, topk_len, dq, dk, dv, workspace,
                                 workspace_bytes, Hq, Nq, Nkv, dqk, dvd, topk, scale, stream,
                                 nullptr, nullptr);
}

const char* attn_last_error(void) { return g_err; }

const char* attn_version(void) { return "attn_mi355x 0.1 (gfx950)"; }

}  // extern "C"
