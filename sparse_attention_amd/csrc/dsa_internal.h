// Internal launcher interface of libdsa (host side).  Each launcher assumes
// its arguments were validated by the C entry points and only enqueues
// kernels on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dsa.h"
#include "launch_plan.h"

namespace dsa {

// Page pool addressing of a paged key or KV store: slot s of sequence r is
// row page * 2^lp + (s mod 2^lp) of the pool, page = table[r * max_pages + (s >> lp)].
struct PageMap {
    const int32_t* table;  // [n_seq, max_pages] device
    int32_t max_pages;
    int32_t lp;       // log2(page size)
    int32_t n_pages;  // pages in the pool
};

// Decode indexer score, one row per sequence (phi = identity).  If zero_words
// > 0 the launch also clears zero_ptr[0 .. zero_words) (the top-k workspace
// header of a fused decode step).
hipError_t launch_score_decode(const void* q, const float* w, const void* k_cache, const float* k_scale,
                               bool key_fp8, const int32_t* positions, int32_t valid_len, int32_t M,
                               int32_t H, int32_t S_max, float scale, float* scores, uint32_t* zero_ptr,
                               size_t zero_words, const PageMap* paging, hipStream_t stream);

// Decode indexer score with a per-head activation (max(0, .)): per-head MFMA, H <= 64.
hipError_t launch_score_decode_heads(const void* q, const float* w, const void* k_cache, const float* k_scale,
                                     bool key_fp8, const int32_t* positions, int32_t valid_len, int32_t M,
                                     int32_t H, int32_t S_max, float scale, float* scores, uint32_t* zero_ptr,
                                     size_t zero_words, const PageMap* paging, hipStream_t stream);

// Prefill indexer score with the identity activation: the heads folded into one
// fp32 query per row (split into bf16 hi + lo MFMA operands); bf16 keys.
hipError_t launch_score_prefill_fold(const void* q, const float* w, const void* k_cache, const int32_t* positions,
                                     int32_t valid_len, int32_t M, int32_t rows_per_seq, int32_t H, int32_t S_max,
                                     float scale, float* scores, hipStream_t stream);

// Prefill indexer score with the per-head activation max(0, .): rows_per_seq
// query rows share one bf16 cache; per-head MFMA, H <= 64.
hipError_t launch_score_prefill(const void* q, const float* w, const void* k_cache, const int32_t* positions,
                                int32_t valid_len, int32_t M, int32_t rows_per_seq, int32_t H, int32_t S_max,
                                float scale, float* scores, hipStream_t stream);

// Top-k per row.  With window > 0 the output row has width k + window and
// holds the top-k with in-window entries replaced by -1, followed by the
// window positions (the decode-step index list).  The workspace holds
// plan::topk_workspace_bytes; header_zeroed: the caller already cleared its
// first plan::topk_header_words words in stream order.
hipError_t launch_topk(const float* scores, int32_t M, int32_t S_max, const int32_t* positions,
                       int32_t valid_len, int32_t k, int32_t window, int32_t* out_idx, float* out_scores,
                       void* workspace, bool header_zeroed, hipStream_t stream);

// The two attention kernels behind launch_sparse_attn (plan::attn_wide
// picks one): many query tokens (128-head workgroups fill the chip; no
// split, no workspace) and few (the list split over workgroups, partial
// results in the workspace, plan::attn_partial_bytes).
hipError_t launch_sparse_attn_wide(const void* q, const void* kv, const float* attn_sink, const int32_t* idx,
                                   int32_t B, int32_t S, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t S_kv,
                                   int32_t K_top, float sm_scale, void* out, float* lse, const PageMap* paging,
                                   hipStream_t stream);
hipError_t launch_sparse_attn_decode(const void* q, const void* kv, const float* attn_sink, const int32_t* idx,
                                     int32_t B, int32_t S, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t S_kv,
                                     int32_t K_top, float sm_scale, void* out, float* lse, void* workspace,
                                     const PageMap* paging, hipStream_t stream);

hipError_t launch_sparse_attn(const void* q, const void* kv, const float* attn_sink, const int32_t* idx,
                              int32_t B, int32_t S, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t S_kv,
                              int32_t K_top, float sm_scale, void* out, float* lse, void* workspace,
                              const PageMap* paging, hipStream_t stream);

// Masked-dense form of launch_sparse_attn: the listed slots of each token
// become a dense list of all S_kv slots (-1 where not selected) in the
// workspace (plan::masked_dense_list_bytes), then the sparse attention runs
// over it (its partials follow the list in the workspace).
hipError_t launch_sparse_attn_masked_dense(const void* q, const void* kv, const float* attn_sink,
                                           const int32_t* topk_idx, int32_t B, int32_t S, int32_t Hq, int32_t Dqk,
                                           int32_t Dv, int32_t S_kv, int32_t K_top, float sm_scale, void* out,
                                           float* lse, void* workspace, hipStream_t stream);

// Key-cache write of T tokens (128 bf16 elements each): fp8 codes + scale,
// bf16 copy, or bf16 quantised and dequantised (qdq).
hipError_t launch_cache_write(const void* k_new, int32_t T, int32_t rows_per_seq, const int32_t* positions,
                              bool key_fp8, bool qdq, bool round_scale, void* k_cache, float* k_scale,
                              int32_t S_max, const PageMap* paging, hipStream_t stream);

// Validates a decode step's arguments as dsa_decode_step does and, when they
// are valid, stores the workspace bytes the step needs in *need.
dsa_status_t decode_step_check(const dsa_decode_args_t* args, size_t* need);

}  // namespace dsa
