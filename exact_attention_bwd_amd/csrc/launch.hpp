// Host-side launchers for the attention kernels.  Arguments are validated by
// the C entry points before these are called; every launch is enqueued on the
// caller's stream and nothing here allocates, frees or synchronises.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace attn {

// BH = B * H query heads; G query heads share each K / V head (H % G == 0)
hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                      int H, int G, int N, int d, bool causal, float scale, hipStream_t stream);

hipError_t launch_bwd_preprocess(const void* o, const void* dO, float* D, int BH, int N, int d,
                                 hipStream_t stream);

size_t bwd_workspace_bytes(int BH, int G, int N, int d, bool causal);

hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                      const float* D, void* dq, void* dk, void* dv, void* workspace, int BH, int H,
                      int G, int N, int d, bool causal, float scale, hipStream_t stream,
                      hipEvent_t main_start = nullptr, hipEvent_t main_stop = nullptr);

// Top-k sparse attention (d_qk = 576, d_v = 512, heads in groups of 64).
size_t sparse_bwd_workspace_bytes(int Hq, int Nq, int Nkv, int topk);

hipError_t launch_sparse_fwd(const void* q, const void* k, const void* v, const int* idx,
                             const int* tlen, void* o, float* lse, int Hq, int Nq, int Nkv,
                             int topk, float scale, hipStream_t stream);

hipError_t launch_sparse_bwd(const void* q, const void* k, const void* v, const void* dO,
                             const float* lse, const float* D, const int* idx, const int* tlen,
                             void* dq, void* dk, void* dv, void* workspace, int Hq, int Nq, int Nkv,
                             int topk, float scale, hipStream_t stream,
                             hipEvent_t main_start = nullptr, hipEvent_t main_stop = nullptr);

}  // namespace attn
