// Host-only stand-ins for the kernel launchers of libdsa, so that the C
// entry points (sparse_attention_amd/csrc/dsa_api.cpp: validation,
// workspace layout, dispatch) and the launch planning they use
// (launch_plan.h, the real one) can be built with AddressSanitizer and
// UndefinedBehaviorSanitizer and driven without a GPU.  Each launcher only
// counts its calls.
#include "dsa_internal.h"

int g_launches = 0;

namespace dsa {

hipError_t launch_score_decode(const void*, const float*, const void*, const float*, bool, const int32_t*, int32_t,
                               int32_t, int32_t, int32_t, float, float*, uint32_t*, size_t, const PageMap*,
                               hipStream_t)
{
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_score_decode_heads(const void*, const float*, const void*, const float*, bool, const int32_t*,
                                     int32_t, int32_t, int32_t, int32_t, float, float*, uint32_t*, size_t,
                                     const PageMap*, hipStream_t)
{
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_sparse_attn_masked_dense(const void*, const void*, const float*, const int32_t*, int32_t, int32_t,
                                           int32_t, int32_t, int32_t, int32_t, int32_t, float, void*, float*, void*,
                                           hipStream_t)
{
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_score_prefill_fold(const void*, const float*, const void*, const int32_t*, int32_t, int32_t,
                                     int32_t, int32_t, int32_t, float, float*, hipStream_t)
{
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_score_prefill(const void*, const float*, const void*, const int32_t*, int32_t, int32_t, int32_t,
                                int32_t, int32_t, float, float*, hipStream_t)
{
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_topk(const float*, int32_t, int32_t, const int32_t*, int32_t, int32_t, int32_t, int32_t*, float*,
                       void*, bool, hipStream_t)
{
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_sparse_attn(const void*, const void*, const float*, const int32_t*, int32_t, int32_t, int32_t,
                              int32_t, int32_t, int32_t, int32_t, float, void*, float*, void*, const PageMap*,
                              hipStream_t)
{
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_cache_write(const void*, int32_t, int32_t, const int32_t*, bool, bool, bool, void*, float*, int32_t,
                              const PageMap*, hipStream_t)
{
    ++g_launches;
    return hipSuccess;
}

}  // namespace dsa
