// Drives every C entry point through its validation paths (host only, built
// with AddressSanitizer): each call must return the documented status, and a
// launcher is reached only when the arguments are valid.  Prints one line per
// failed expectation and "ok <n>" at the end.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/attn_mi355x.h"

extern int g_launches;
static int g_fail = 0, g_checks = 0;

static void expect(const char* what, int got, int want, int launches_before, bool launched) {
    ++g_checks;
    const bool did = g_launches != launches_before;
    if (got != want || did != launched) {
        ++g_fail;
        printf("FAIL %s: status %d (want %d), launched %d (want %d): %s\n", what, got, want, (int)did,
               (int)launched, attn_last_error());
    }
    if (got != 0 && strlen(attn_last_error()) == 0) {
        ++g_fail;
        printf("FAIL %s: no message for status %d\n", what, got);
    }
}

#define CHECK(what, call, want, launched)          \
    do {                                           \
        int before = g_launches;                   \
        int st = (call);                           \
        expect(what, st, want, before, launched);  \
    } while (0)

int main() {
    alignas(256) static char buf[1 << 16];
    void* p = buf;                                   // any aligned address: nothing is launched
    void* mis = buf + 2;                             // not 16-byte aligned
    float* f = (float*)(buf + 4096);
    int* ip = (int*)(buf + 8192);
    const float nan = NAN, inf = INFINITY;

    // forward
    CHECK("fwd ok", attn_fwd(p, p, p, p, f, 1, 2, 64, 128, 1, 0.1f, nullptr), 0, true);
    CHECK("fwd null q", attn_fwd(nullptr, p, p, p, f, 1, 2, 64, 128, 1, 0.1f, nullptr), ATTN_ERR_INVALID_ARG, false);
    CHECK("fwd misaligned v", attn_fwd(p, p, mis, p, f, 1, 2, 64, 128, 1, 0.1f, nullptr), ATTN_ERR_INVALID_ARG, false);
    CHECK("fwd d=96", attn_fwd(p, p, p, p, f, 1, 2, 64, 96, 1, 0.1f, nullptr), ATTN_ERR_UNSUPPORTED, false);
    CHECK("fwd negative N", attn_fwd(p, p, p, p, f, 1, 2, -1, 64, 1, 0.1f, nullptr), ATTN_ERR_INVALID_ARG, false);
    CHECK("fwd nan scale", attn_fwd(p, p, p, p, f, 1, 2, 64, 64, 1, nan, nullptr), ATTN_ERR_INVALID_ARG, false);
    CHECK("fwd inf scale", attn_fwd(p, p, p, p, f, 1, 2, 64, 64, 1, inf, nullptr), ATTN_ERR_INVALID_ARG, false);
    CHECK("fwd empty", attn_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 2, 64, 64, 1, 0.1f, nullptr), 0, false);
    CHECK("fwd huge", attn_fwd(p, p, p, p, f, 1 << 20, 1 << 10, 1 << 20, 64, 1, 0.1f, nullptr), ATTN_ERR_UNSUPPORTED, false);
    CHECK("fwd_gqa Hkv=3 of 4", attn_fwd_gqa(p, p, p, p, f, 1, 4, 3, 64, 64, 0, 0.1f, nullptr), ATTN_ERR_INVALID_ARG, false);
    CHECK("fwd_gqa ok", attn_fwd_gqa(p, p, p, p, f, 1, 4, 2, 64, 64, 0, 0.1f, nullptr), 0, true);
    // preprocess
    CHECK("pre ok", attn_bwd_preprocess(p, p, f, 1, 2, 64, 128, nullptr), 0, true);
    CHECK("pre d=512", attn_bwd_preprocess(p, p, f, 1, 64, 64, 512, nullptr), 0, true);
    CHECK("pre null D", attn_bwd_preprocess(p, p, nullptr, 1, 2, 64, 128, nullptr), ATTN_ERR_INVALID_ARG, false);
    CHECK("pre misaligned D", attn_bwd_preprocess(p, p, (float*)(buf + 1), 1, 2, 64, 128, nullptr), ATTN_ERR_INVALID_ARG, false);
    // backward
    const size_t need = attn_bwd_workspace_bytes_ex(1, 2, 2, 64, 128, 1);
    if (need == 0 || need > sizeof(buf)) {
        printf("FAIL workspace size %zu\n", need);
        ++g_fail;
    }
    CHECK("bwd ok", attn_bwd(p, p, p, p, f, f, p, p, p, p, need, 1, 2, 64, 128, 1, 0.1f, nullptr), 0, true);
    CHECK("bwd ws small", attn_bwd(p, p, p, p, f, f, p, p, p, p, need - 1, 1, 2, 64, 128, 1, 0.1f, nullptr),
          ATTN_ERR_WORKSPACE, false);
    CHECK("bwd ws null", attn_bwd(p, p, p, p, f, f, p, p, p, nullptr, need, 1, 2, 64, 128, 1, 0.1f, nullptr),
          ATTN_ERR_INVALID_ARG, false);
    CHECK("bwd ws misaligned", attn_bwd(p, p, p, p, f, f, p, p, p, mis, need, 1, 2, 64, 128, 1, 0.1f, nullptr),
          ATTN_ERR_INVALID_ARG, false);
    CHECK("bwd null dk", attn_bwd(p, p, p, p, f, f, p, nullptr, p, p, need, 1, 2, 64, 128, 1, 0.1f, nullptr),
          ATTN_ERR_INVALID_ARG, false);
    CHECK("bwd null lse", attn_bwd(p, p, p, p, nullptr, f, p, p, p, p, need, 1, 2, 64, 128, 1, 0.1f, nullptr),
          ATTN_ERR_INVALID_ARG, false);
    CHECK("bwd d=32", attn_bwd(p, p, p, p, f, f, p, p, p, p, need, 1, 2, 64, 32, 1, 0.1f, nullptr),
          ATTN_ERR_UNSUPPORTED, false);
    CHECK("bwd nan scale", attn_bwd(p, p, p, p, f, f, p, p, p, p, need, 1, 2, 64, 128, 1, nan, nullptr),
          ATTN_ERR_INVALID_ARG, false);
    CHECK("bwd empty", attn_bwd(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                nullptr, 0, 1, 0, 64, 128, 1, 0.1f, nullptr), 0, false);
    CHECK("bwd_timed ok", attn_bwd_timed(p, p, p, p, f, f, p, p, p, p, need, 1, 2, 64, 128, 1, 0.1f, nullptr,
                                         nullptr, nullptr), 0, true);
    CHECK("bwd_gqa Hkv=0", attn_bwd_gqa(p, p, p, p, f, f, p, p, p, p, need, 1, 2, 0, 64, 128, 1, 0.1f, nullptr),
          ATTN_ERR_INVALID_ARG, false);
    if (attn_bwd_workspace_bytes(1, 2, 64, 96) != 0 || attn_bwd_workspace_bytes_ex(1, 4, 3, 64, 64, 0) != 0) {
        printf("FAIL workspace size of an unsupported shape is not 0\n");
        ++g_fail;
    }
    // sparse
    const size_t sneed = attn_sparse_bwd_workspace_bytes(64, 16, 16, 576, 512, 8);
    CHECK("sfwd ok", attn_sparse_fwd(p, p, p, ip, nullptr, p, f, 64, 16, 16, 576, 512, 8, 0.1f, nullptr), 0, true);
    CHECK("sfwd d_qk=128", attn_sparse_fwd(p, p, p, ip, nullptr, p, f, 64, 16, 16, 128, 512, 8, 0.1f, nullptr),
          ATTN_ERR_UNSUPPORTED, false);
    CHECK("sfwd Hq=32", attn_sparse_fwd(p, p, p, ip, nullptr, p, f, 32, 16, 16, 576, 512, 8, 0.1f, nullptr),
          ATTN_ERR_UNSUPPORTED, false);
    CHECK("sfwd null idx", attn_sparse_fwd(p, p, p, nullptr, nullptr, p, f, 64, 16, 16, 576, 512, 8, 0.1f, nullptr),
          ATTN_ERR_INVALID_ARG, false);
    CHECK("sfwd misaligned idx", attn_sparse_fwd(p, p, p, (int*)(buf + 2), nullptr, p, f, 64, 16, 16, 576, 512, 8,
                                                 0.1f, nullptr), ATTN_ERR_INVALID_ARG, false);
    CHECK("sbwd ok", attn_sparse_bwd(p, p, p, p, f, f, ip, ip, p, p, p, p, sneed, 64, 16, 16, 576, 512, 8, 0.1f,
                                     nullptr), 0, true);
    CHECK("sbwd ws small", attn_sparse_bwd(p, p, p, p, f, f, ip, ip, p, p, p, p, sneed - 1, 64, 16, 16, 576, 512, 8,
                                           0.1f, nullptr), ATTN_ERR_WORKSPACE, false);
    CHECK("sbwd Nkv too large", attn_sparse_bwd(p, p, p, p, f, f, ip, ip, p, p, p, p, sneed, 64, 16, 20000, 576,
                                                512, 8, 0.1f, nullptr), ATTN_ERR_UNSUPPORTED, false);
    CHECK("sbwd negative topk", attn_sparse_bwd(p, p, p, p, f, f, ip, ip, p, p, p, p, sneed, 64, 16, 16, 576, 512,
                                                -1, 0.1f, nullptr), ATTN_ERR_INVALID_ARG, false);
    if (strlen(attn_version()) == 0) {
        printf("FAIL empty version\n");
        ++g_fail;
    }
    printf("%s %d\n", g_fail ? "failed" : "ok", g_checks);
    return g_fail ? 1 : 0;
}
