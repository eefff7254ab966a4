// Masked-dense form of the top-k sparse attention, for short sequences, on gfx950.
//
// Definition (OpenXLA tokamax "Supported Ops and Hardware", Attention
// Variants table, masked_dense_mla row: multi-head latent attention
// restricted to a selected top-k subset of the KV positions through a dense
// mask, the form used for shorter sequences).  The attention itself is the
// one of the sparse path (softmax with the sink term, NeMo AutoModel
// deepseek_v4 optimized_kernels page, sparse_attention_torch); the listed
// positions only select which slots enter it, each at most once.
//
// The mask is made dense over the sequence's S_kv slots: a list of every
// slot in slot order, with -1 where the slot is not selected.  The sparse
// attention kernels then walk the whole sequence: their 32-row blocks are
// runs of consecutive rows (contiguous copies into LDS, no index-driven
// gather), and the unselected slots are masked as any -1 entry is.  The
// cost grows with S_kv, not with the list length, so this form pays only
// when the selection covers a large part of a short sequence.
#include "device_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;

// One workgroup per query token: the listed slots as a bitmap in LDS
// (S_kv bits), then the dense list written in slot order.
__global__ __launch_bounds__(kThreads) void masked_dense_list_kernel(const int32_t* __restrict__ idx, int32_t K_top,
                                                                     int32_t S_kv, int32_t* __restrict__ dense)
{
    extern __shared__ uint32_t bits[];
    const int nw = (S_kv + 31) >> 5;
    const size_t bs = blockIdx.x;
    for (int i = threadIdx.x; i < nw; i += kThreads) bits[i] = 0u;
    __syncthreads();
    const int32_t* __restrict__ il = idx + bs * K_top;
    for (int j = threadIdx.x; j < K_top; j += kThreads) {
        const int p = il[j];
        if (p >= 0 && p < S_kv) atomicOr(&bits[p >> 5], 1u << (p & 31));
    }
    __syncthreads();
    int32_t* __restrict__ o = dense + bs * S_kv;
    for (int p = threadIdx.x; p < S_kv; p += kThreads) o[p] = ((bits[p >> 5] >> (p & 31)) & 1u) ? p : -1;
}

}  // namespace

hipError_t launch_sparse_attn_masked_dense(const void* q, const void* kv, const float* attn_sink,
                                           const int32_t* topk_idx, int32_t B, int32_t S, int32_t Hq, int32_t Dqk,
                                           int32_t Dv, int32_t S_kv, int32_t K_top, float sm_scale, void* out,
                                           float* lse, void* workspace, hipStream_t stream)
{
    int32_t* dense = static_cast<int32_t*>(workspace);
    const size_t lds = (size_t)((S_kv + 31) / 32) * 4;
    masked_dense_list_kernel<<<B * S, kThreads, lds, stream>>>(topk_idx, K_top, S_kv, dense);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    void* attn_ws = static_cast<char*>(workspace) + plan::masked_dense_list_bytes(B, S, S_kv);
    return launch_sparse_attn(q, kv, attn_sink, dense, B, S, Hq, Dqk, Dv, S_kv, S_kv, sm_scale, out, lse, attn_ws,
                              nullptr, stream);
}

}  // namespace dsa
