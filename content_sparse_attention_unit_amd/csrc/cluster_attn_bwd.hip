// cluster_attn_bwd.hip -- backward of the in-cluster attention (gfx950).
#include "rt_common.hpp"
#include "rt_internal.hpp"

namespace rt {

size_t bwd_workspace_bytes(int BH, int n, int d, int k, int w) {
    (void)BH; (void)n; (void)d; (void)k; (void)w;
    return 0;
}

hipError_t launch_cluster_attn_bwd(const void*, const void*, const void*, int, const float*,
                                   const float*, const int32_t*, const float*, const void*, int,
                                   int, int, int, int, float, int, float*, float*, float*, float*,
                                   hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace rt
