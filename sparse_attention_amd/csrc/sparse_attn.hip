// Top-k sparse multi-query attention with an attention sink: choice of kernel
// (NeMo AutoModel deepseek_v4 optimized_kernels page, sparse_attention_torch;
// kwkr.cn article on DeepSeek-V4-Pro inference/kernel.py, sparse-attention
// section).
//
// Calls whose tokens fill the chip with 128-head workgroups (prefill-shaped)
// run sparse_attn_wide.hip: 32 heads per wave, 64-entry blocks, no split of
// the list.  Calls with fewer tokens (decode) run sparse_attn_decode.hip:
// 16 heads per wave, 64-head workgroups, the list split over workgroups and
// merged by a combine kernel.  Both compute the same function; the choice is
// by measured speed on the two regimes.
#include "dsa_internal.h"

namespace dsa {

hipError_t launch_sparse_attn(const void* q, const void* kv, const float* attn_sink, const int32_t* idx,
                              int32_t B, int32_t S, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t S_kv,
                              int32_t K_top, float sm_scale, void* out, float* lse, void* workspace,
                              const PageMap* paging, hipStream_t stream)
{
    if (plan::attn_wide(B, S, Hq))
        return launch_sparse_attn_wide(q, kv, attn_sink, idx, B, S, Hq, Dqk, Dv, S_kv, K_top, sm_scale, out, lse,
                                       paging, stream);
    return launch_sparse_attn_decode(q, kv, attn_sink, idx, B, S, Hq, Dqk, Dv, S_kv, K_top, sm_scale, out, lse,
                                     workspace, paging, stream);
}

}  // namespace dsa
