// Stand-ins for the kernel launchers, for a host-only build of the C entry
// points (argument validation): each records that it was reached and
// launches nothing.
#include "../../exact_attention_bwd_amd/csrc/launch.hpp"

int g_launches = 0;

namespace attn {

hipError_t launch_fwd(const void*, const void*, const void*, void*, float*, int, int, int, int, int, bool,
                      float, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_bwd_preprocess(const void*, const void*, float*, int, int, int, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}

size_t bwd_workspace_bytes(int BH, int G, int N, int d, bool causal) {
    return (size_t)BH * N * d * (causal ? 3 : 4) / G + 256;
}

hipError_t launch_bwd(const void*, const void*, const void*, const void*, const float*, const float*, void*,
                      void*, void*, void*, int, int, int, int, int, bool, float, hipStream_t, hipEvent_t,
                      hipEvent_t) {
    ++g_launches;
    return hipSuccess;
}

size_t sparse_bwd_workspace_bytes(int Hq, int Nq, int Nkv, int topk) {
    return (size_t)Hq * Nq + (size_t)Nkv * topk + 256;
}

hipError_t launch_sparse_fwd(const void*, const void*, const void*, const int*, const int*, void*, float*, int,
                             int, int, int, float, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_sparse_bwd(const void*, const void*, const void*, const void*, const float*, const float*,
                             const int*, const int*, void*, void*, void*, void*, int, int, int, int, float,
                             hipStream_t, hipEvent_t, hipEvent_t) {
    ++g_launches;
    return hipSuccess;
}

}  // namespace attn
