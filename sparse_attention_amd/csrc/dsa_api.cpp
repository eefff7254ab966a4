// C entry points of libdsa: host-side validation, workspace carving and
// dispatch to the gfx950 kernels.  Validation completes before anything is
// enqueued, so an error status leaves every output untouched.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include <climits>
#include <cstddef>

#include "dsa.h"
#include "dsa_internal.h"

namespace {

constexpr size_t kAlign = 256;  // workspace sub-buffer alignment

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

dsa_status_t launch_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH; }

dsa_status_t check_index_score(const void* q, const float* w, const void* k_cache, const float* k_scale,
                               dsa_key_dtype_t k_dtype, int32_t M, int32_t rows_per_seq, int32_t H, int32_t D,
                               int32_t S_max, uint32_t flags, const float* scores)
{
    if (!q || !w || !k_cache || !scores) return DSA_ERR_NULL;
    if (k_dtype != DSA_KEY_BF16 && k_dtype != DSA_KEY_FP8_E4M3) return DSA_ERR_UNSUPPORTED;
    if (k_dtype == DSA_KEY_FP8_E4M3 && !k_scale) return DSA_ERR_NULL;
    if (k_dtype == DSA_KEY_BF16 && k_scale) return DSA_ERR_SHAPE;
    if (M < 1 || rows_per_seq < 1 || H < 1 || S_max < 1) return DSA_ERR_SHAPE;
    if (M % rows_per_seq != 0) return DSA_ERR_SHAPE;
    if (D != DSA_INDEX_HEAD_DIM) return DSA_ERR_UNSUPPORTED;
    if (H > 128) return DSA_ERR_UNSUPPORTED;
    if (flags & ~DSA_SCORE_RELU) return DSA_ERR_UNSUPPORTED;
    if (rows_per_seq == 1) {
        if ((flags & DSA_SCORE_RELU) && H > 64) return DSA_ERR_UNSUPPORTED;  // per-head MFMA path: 4 head tiles
        if (M > 65535) return DSA_ERR_SHAPE;
    } else {
        if (k_dtype != DSA_KEY_BF16) return DSA_ERR_UNSUPPORTED;
        if ((flags & DSA_SCORE_RELU) && H > 64) return DSA_ERR_UNSUPPORTED;  // per-head MFMA path: 4 head tiles
        if ((long long)S_max * D * 2 > INT32_MAX) return DSA_ERR_SHAPE;  // one sequence's keys: 32-bit offsets
    }
    if (!aligned16(q) || !aligned16(k_cache)) return DSA_ERR_ALIGN;
    if (!aligned16(w) || !aligned16(scores) || (k_scale && !aligned16(k_scale))) return DSA_ERR_ALIGN;
    return DSA_OK;
}

dsa_status_t check_topk(const float* scores, int32_t M, int32_t S_max, int32_t k, const int32_t* topk_idx)
{
    if (!scores || !topk_idx) return DSA_ERR_NULL;
    if (M < 1 || S_max < 1 || S_max > DSA_MAX_TOPK_SLOTS) return DSA_ERR_SHAPE;
    if (k < 1 || k > DSA_MAX_TOPK) return DSA_ERR_UNSUPPORTED;
    if (!aligned16(scores) || !aligned16(topk_idx)) return DSA_ERR_ALIGN;
    return DSA_OK;
}

dsa_status_t check_sparse_attn(const void* q, const void* kv, const int32_t* idx, int32_t B, int32_t S, int32_t Hq,
                               int32_t Dqk, int32_t Dv, int32_t S_kv, int32_t K_top, const void* out, bool paged = false)
{
    if (!q || !kv || !idx || !out) return DSA_ERR_NULL;
    if (B < 1 || S < 1 || Hq < 1 || S_kv < 1 || K_top < 1 || Hq > DSA_MAX_ATTN_HEADS) return DSA_ERR_SHAPE;
    if (Dqk < 32 || Dqk > DSA_MAX_ATTN_DIM || Dqk % 32 != 0) return DSA_ERR_UNSUPPORTED;
    if (Dv < 16 || Dv > Dqk || Dv > DSA_MAX_ATTN_VDIM || Dv % 16 != 0) return DSA_ERR_UNSUPPORTED;
    if ((long long)B * S > 65535) return DSA_ERR_SHAPE;
    if (!paged && (long long)S_kv * Dqk * 2 > INT32_MAX) return DSA_ERR_SHAPE;  // one sequence's KV: 32-bit offsets
    if (!aligned16(q) || !aligned16(kv) || !aligned16(out)) return DSA_ERR_ALIGN;
    return DSA_OK;
}

// A paged-cache descriptor covering n_slots logical slots per sequence, as
// the kernels' page map.
dsa_status_t check_paging(const dsa_paged_cache_t* pg, int32_t n_slots, dsa::PageMap* pm)
{
    if (!pg || !pg->block_table) return DSA_ERR_NULL;
    const int32_t P = pg->page_size;
    if (P < 64 || P > 65536 || (P & (P - 1)) != 0) return DSA_ERR_UNSUPPORTED;
    if (pg->max_pages < 1 || pg->n_pages < 1) return DSA_ERR_SHAPE;
    if ((long long)pg->n_pages * P > INT32_MAX) return DSA_ERR_SHAPE;  // pool rows: 31-bit indices
    if ((long long)n_slots > (long long)pg->max_pages * P) return DSA_ERR_SHAPE;
    if (!aligned16(pg->block_table)) return DSA_ERR_ALIGN;
    int lp = 0;
    while ((1 << lp) < P) ++lp;
    *pm = dsa::PageMap{pg->block_table, pg->max_pages, lp, pg->n_pages};
    return DSA_OK;
}

struct decode_layout {
    size_t scores_off, scores_bytes;
    size_t topk_off, topk_bytes;
    size_t list_off, list_bytes;
    size_t attn_off, attn_bytes;
    size_t total;
};

decode_layout layout_decode(const dsa_decode_args_t* a)
{
    decode_layout L{};
    size_t off = 0;
    L.scores_bytes = a->scores ? 0 : (size_t)a->B * a->S_max * sizeof(float);
    L.scores_off = off;
    off += round_up(L.scores_bytes);
    L.topk_bytes = dsa::plan::topk_workspace_bytes(a->B, a->S_max);
    L.topk_off = off;
    off += round_up(L.topk_bytes);
    const int32_t K_top = a->index_topk + a->window;
    L.list_bytes = a->index_list ? 0 : (size_t)a->B * K_top * sizeof(int32_t);
    L.list_off = off;
    off += round_up(L.list_bytes);
    L.attn_bytes = dsa::plan::attn_partial_bytes(a->B, 1, a->Hq, a->Dv, K_top);
    L.attn_off = off;
    off += round_up(L.attn_bytes);
    L.total = off;
    return L;
}

// index_flags / paging, or 0 / NULL for a struct that ends before the field
uint32_t decode_flags(const dsa_decode_args_t* a)
{
    return a->struct_size >= offsetof(dsa_decode_args_t, index_flags) + sizeof(uint32_t) ? a->index_flags : 0u;
}
const dsa_paged_cache_t* decode_paging(const dsa_decode_args_t* a)
{
    return a->struct_size >= offsetof(dsa_decode_args_t, paging) + sizeof(void*) ? a->paging : nullptr;
}

dsa_status_t check_decode(const dsa_decode_args_t* a)
{
    if (!a) return DSA_ERR_NULL;
    if (a->struct_size < offsetof(dsa_decode_args_t, index_flags)) return DSA_ERR_UNSUPPORTED;
    const uint32_t flags = decode_flags(a);
    if (flags & ~DSA_SCORE_RELU) return DSA_ERR_UNSUPPORTED;
    if ((flags & DSA_SCORE_RELU) && a->H > 64) return DSA_ERR_UNSUPPORTED;
    if (!a->index_q || !a->index_w || !a->k_cache || !a->q || !a->kv || !a->out) return DSA_ERR_NULL;
    if (a->k_dtype != DSA_KEY_BF16 && a->k_dtype != DSA_KEY_FP8_E4M3) return DSA_ERR_UNSUPPORTED;
    if (a->k_dtype == DSA_KEY_FP8_E4M3 && !a->k_scale) return DSA_ERR_NULL;
    if (a->k_dtype == DSA_KEY_BF16 && a->k_scale) return DSA_ERR_SHAPE;
    if (a->B < 1 || a->B > 65535 || a->H < 1 || a->S_max < 1 || a->S_max > DSA_MAX_TOPK_SLOTS) return DSA_ERR_SHAPE;
    if (a->H > 128) return DSA_ERR_UNSUPPORTED;
    if (a->index_topk < 1 || a->index_topk > DSA_MAX_TOPK) return DSA_ERR_UNSUPPORTED;
    if (a->window < 0 || a->window > a->S_max) return DSA_ERR_SHAPE;
    if (a->Hq < 1 || a->Hq > DSA_MAX_ATTN_HEADS) return DSA_ERR_SHAPE;
    if (a->Dqk < 32 || a->Dqk > DSA_MAX_ATTN_DIM || a->Dqk % 32 != 0) return DSA_ERR_UNSUPPORTED;
    if (a->Dv < 16 || a->Dv > a->Dqk || a->Dv > DSA_MAX_ATTN_VDIM || a->Dv % 16 != 0) return DSA_ERR_UNSUPPORTED;
    if (decode_paging(a)) {
        dsa::PageMap pm;
        const dsa_status_t ps = check_paging(decode_paging(a), a->S_max, &pm);
        if (ps != DSA_OK) return ps;
    } else if ((long long)a->S_max * a->Dqk * 2 > INT32_MAX) {
        return DSA_ERR_SHAPE;  // one sequence's KV rows: 32-bit offsets
    }
    if (!aligned16(a->index_q) || !aligned16(a->index_w) || !aligned16(a->k_cache) || !aligned16(a->q) ||
        !aligned16(a->kv) || !aligned16(a->out))
        return DSA_ERR_ALIGN;
    if ((a->k_scale && !aligned16(a->k_scale)) || (a->scores && !aligned16(a->scores)) ||
        (a->index_list && !aligned16(a->index_list)))
        return DSA_ERR_ALIGN;
    return DSA_OK;
}

dsa_status_t check_cache_write(const void* k_new, int32_t T, int32_t rows_per_seq, int32_t D,
                               const int32_t* positions, dsa_key_dtype_t k_dtype, const void* k_cache,
                               const float* k_scale, int32_t S_max, uint32_t flags)
{
    if (!k_cache || (T != 0 && (!k_new || !positions))) return DSA_ERR_NULL;
    if (k_dtype != DSA_KEY_BF16 && k_dtype != DSA_KEY_FP8_E4M3) return DSA_ERR_UNSUPPORTED;
    if (k_dtype == DSA_KEY_FP8_E4M3 && !k_scale) return DSA_ERR_NULL;
    if (k_dtype == DSA_KEY_BF16 && k_scale) return DSA_ERR_SHAPE;
    if (T < 0 || rows_per_seq < 1 || S_max < 1 || T % rows_per_seq != 0) return DSA_ERR_SHAPE;
    if (D != DSA_INDEX_HEAD_DIM) return DSA_ERR_UNSUPPORTED;
    if (flags & ~(DSA_CACHE_ROUND_SCALE | DSA_CACHE_QDQ)) return DSA_ERR_UNSUPPORTED;
    const bool qdq = (flags & DSA_CACHE_QDQ) != 0;
    if (qdq && k_dtype != DSA_KEY_BF16) return DSA_ERR_UNSUPPORTED;
    if ((flags & DSA_CACHE_ROUND_SCALE) && k_dtype == DSA_KEY_BF16 && !qdq) return DSA_ERR_UNSUPPORTED;
    if (!aligned16(k_new) || !aligned16(k_cache) || !aligned16(positions) || (k_scale && !aligned16(k_scale)))
        return DSA_ERR_ALIGN;
    return DSA_OK;
}

}  // namespace

dsa_status_t dsa::decode_step_check(const dsa_decode_args_t* args, size_t* need)
{
    const dsa_status_t s = check_decode(args);
    if (s == DSA_OK) *need = layout_decode(args).total;
    return s;
}

extern "C" {

const char* dsa_version(void) { return "0.1.0"; }

const char* dsa_status_string(dsa_status_t status)
{
    switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_NULL: return "DSA_ERR_NULL: a required pointer is NULL";
    case DSA_ERR_SHAPE: return "DSA_ERR_SHAPE: a size is out of range or inconsistent";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: request not implemented by this build";
    case DSA_ERR_ALIGN: return "DSA_ERR_ALIGN: a pointer is not 16-byte aligned";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing or too small";
    case DSA_ERR_LAUNCH: return "DSA_ERR_LAUNCH: kernel launch failed";
    }
    return "unknown dsa_status_t";
}

float dsa_mask_bound(void) { return -0x1.FEp+127f; }

dsa_status_t dsa_index_score(const void* q, const float* w, const void* k_cache, const float* k_scale,
                             dsa_key_dtype_t k_dtype, const int32_t* positions, int32_t valid_len, int32_t M,
                             int32_t rows_per_seq, int32_t H, int32_t D, int32_t S_max, float scale,
                             uint32_t flags, float* scores, hipStream_t stream)
{
    dsa_status_t s = check_index_score(q, w, k_cache, k_scale, k_dtype, M, rows_per_seq, H, D, S_max, flags, scores);
    if (s != DSA_OK) return s;
    if (rows_per_seq == 1 && (flags & DSA_SCORE_RELU))
        return launch_status(dsa::launch_score_decode_heads(q, w, k_cache, k_scale, k_dtype == DSA_KEY_FP8_E4M3,
                                                            positions, valid_len, M, H, S_max, scale, scores, nullptr, 0,
                                                            nullptr, stream));
    if (rows_per_seq == 1)
        return launch_status(dsa::launch_score_decode(q, w, k_cache, k_scale, k_dtype == DSA_KEY_FP8_E4M3, positions,
                                                      valid_len, M, H, S_max, scale, scores, nullptr, 0, nullptr,
                                                      stream));
    // prefill: with the identity activation the heads fold into one query per
    // row (bound by the score writes); ReLU needs the per-head MFMA contraction
    if (!(flags & DSA_SCORE_RELU))
        return launch_status(dsa::launch_score_prefill_fold(q, w, k_cache, positions, valid_len, M, rows_per_seq, H,
                                                            S_max, scale, scores, stream));
    return launch_status(dsa::launch_score_prefill(q, w, k_cache, positions, valid_len, M, rows_per_seq, H, S_max,
                                                   scale, scores, stream));
}

size_t dsa_topk_workspace_size(int32_t M, int32_t S_max, int32_t index_topk)
{
    (void)index_topk;
    if (M < 1 || S_max < 1) return 0;
    return dsa::plan::topk_workspace_bytes(M, S_max);
}

dsa_status_t dsa_topk(const float* scores, int32_t M, int32_t S_max, const int32_t* positions, int32_t valid_len,
                      int32_t index_topk, int32_t* topk_idx, float* topk_scores, void* workspace,
                      size_t workspace_bytes, hipStream_t stream)
{
    dsa_status_t s = check_topk(scores, M, S_max, index_topk, topk_idx);
    if (s != DSA_OK) return s;
    const size_t need = dsa::plan::topk_workspace_bytes(M, S_max);
    if (need > 0 && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE;
    if (need > 0 && !aligned16(workspace)) return DSA_ERR_ALIGN;
    return launch_status(dsa::launch_topk(scores, M, S_max, positions, valid_len, index_topk, 0, topk_idx,
                                          topk_scores, workspace, false, stream));
}

size_t dsa_sparse_attn_workspace_size(int32_t B, int32_t S, int32_t Hq, int32_t Dv, int32_t K_top)
{
    if (B < 1 || S < 1 || Hq < 1 || Dv < 1 || K_top < 1) return 0;
    if ((long long)B * S > 65535 || Hq > DSA_MAX_ATTN_HEADS || Dv > DSA_MAX_ATTN_VDIM) return 0;  // rejected by the call
    return dsa::plan::attn_partial_bytes(B, S, Hq, Dv, K_top);
}

dsa_status_t dsa_sparse_attn(const void* q, const void* kv, const float* attn_sink, const int32_t* topk_idx, int32_t B,
                             int32_t S, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t S_kv, int32_t K_top,
                             float sm_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                             hipStream_t stream)
{
    dsa_status_t s = check_sparse_attn(q, kv, topk_idx, B, S, Hq, Dqk, Dv, S_kv, K_top, out);
    if (s != DSA_OK) return s;
    const size_t need = dsa::plan::attn_partial_bytes(B, S, Hq, Dv, K_top);
    if (need > 0 && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE;
    if (need > 0 && !aligned16(workspace)) return DSA_ERR_ALIGN;
    return launch_status(dsa::launch_sparse_attn(q, kv, attn_sink, topk_idx, B, S, Hq, Dqk, Dv, S_kv, K_top, sm_scale,
                                                 out, lse, workspace, nullptr, stream));
}

size_t dsa_sparse_attn_masked_dense_workspace_size(int32_t B, int32_t S, int32_t Hq, int32_t Dv, int32_t S_kv)
{
    if (B < 1 || S < 1 || Hq < 1 || Hq > DSA_MAX_ATTN_HEADS || Dv < 1 || Dv > DSA_MAX_ATTN_VDIM || S_kv < 1 ||
        S_kv > DSA_MASKED_DENSE_MAX_SLOTS || (long long)B * S > 65535)
        return 0;
    return dsa::plan::masked_dense_workspace_bytes(B, S, Hq, Dv, S_kv);
}

dsa_status_t dsa_sparse_attn_masked_dense(const void* q, const void* kv, const float* attn_sink,
                                          const int32_t* topk_idx, int32_t B, int32_t S, int32_t Hq, int32_t Dqk,
                                          int32_t Dv, int32_t S_kv, int32_t K_top, float sm_scale, void* out,
                                          float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    dsa_status_t s = check_sparse_attn(q, kv, topk_idx, B, S, Hq, Dqk, Dv, S_kv, K_top, out);
    if (s != DSA_OK) return s;
    if (S_kv > DSA_MASKED_DENSE_MAX_SLOTS) return DSA_ERR_SHAPE;
    const size_t need = dsa::plan::masked_dense_workspace_bytes(B, S, Hq, Dv, S_kv);
    if (!workspace || workspace_bytes < need) return DSA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return DSA_ERR_ALIGN;
    return launch_status(dsa::launch_sparse_attn_masked_dense(q, kv, attn_sink, topk_idx, B, S, Hq, Dqk, Dv, S_kv,
                                                              K_top, sm_scale, out, lse, workspace, stream));
}

size_t dsa_decode_step_workspace_size(const dsa_decode_args_t* args)
{
    // shapes the step would reject give 0 (pointers are not needed for the size)
    if (!args || args->struct_size < offsetof(dsa_decode_args_t, index_flags) || args->B < 1 || args->B > 65535 ||
        args->S_max < 1 || args->S_max > DSA_MAX_TOPK_SLOTS || args->index_topk < 1 ||
        args->index_topk > DSA_MAX_TOPK || args->window < 0 || args->window > args->S_max || args->Hq < 1 ||
        args->Hq > DSA_MAX_ATTN_HEADS || args->Dv < 1 || args->Dv > DSA_MAX_ATTN_VDIM)
        return 0;
    return layout_decode(args).total;
}

dsa_status_t dsa_decode_step(const dsa_decode_args_t* args, void* workspace, size_t workspace_bytes,
                             hipStream_t stream)
{
    dsa_status_t s = check_decode(args);
    if (s != DSA_OK) return s;
    const decode_layout L = layout_decode(args);
    if (L.total > 0 && (!workspace || workspace_bytes < L.total)) return DSA_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    float* scores = args->scores ? args->scores : reinterpret_cast<float*>(ws + L.scores_off);
    int32_t* list = args->index_list ? args->index_list : reinterpret_cast<int32_t*>(ws + L.list_off);
    void* attn_ws = L.attn_bytes ? static_cast<void*>(ws + L.attn_off) : nullptr;
    void* topk_ws = L.topk_bytes ? static_cast<void*>(ws + L.topk_off) : nullptr;
    const int32_t K_top = args->index_topk + args->window;

    const bool relu = (decode_flags(args) & DSA_SCORE_RELU) != 0;
    dsa::PageMap pm_store;
    const dsa::PageMap* pm = nullptr;
    if (decode_paging(args)) {
        check_paging(decode_paging(args), args->S_max, &pm_store);  // validated by check_decode
        pm = &pm_store;
    }
    hipError_t e;
    // either scorer also clears the top-k workspace header, saving a launch
    if (relu) {
        e = dsa::launch_score_decode_heads(args->index_q, args->index_w, args->k_cache, args->k_scale,
                                           args->k_dtype == DSA_KEY_FP8_E4M3, args->positions, args->valid_len,
                                           args->B, args->H, args->S_max, args->index_scale, scores,
                                           static_cast<uint32_t*>(topk_ws),
                                           dsa::plan::topk_header_words(args->B, args->S_max), pm, stream);
    } else {
        e = dsa::launch_score_decode(args->index_q, args->index_w, args->k_cache, args->k_scale,
                                     args->k_dtype == DSA_KEY_FP8_E4M3, args->positions, args->valid_len, args->B,
                                     args->H, args->S_max, args->index_scale, scores, static_cast<uint32_t*>(topk_ws),
                                     dsa::plan::topk_header_words(args->B, args->S_max), pm, stream);
    }
    if (e != hipSuccess) return DSA_ERR_LAUNCH;
    e = dsa::launch_topk(scores, args->B, args->S_max, args->positions, args->valid_len, args->index_topk,
                         args->window, list, nullptr, topk_ws, true, stream);
    if (e != hipSuccess) return DSA_ERR_LAUNCH;
    e = dsa::launch_sparse_attn(args->q, args->kv, args->attn_sink, list, args->B, 1, args->Hq, args->Dqk, args->Dv,
                                args->S_max, K_top, args->sm_scale, args->out, args->lse, attn_ws, pm, stream);
    return launch_status(e);
}

dsa_status_t dsa_index_score_paged(const void* q, const float* w, const void* k_pool, const float* k_scale_pool,
                                   dsa_key_dtype_t k_dtype, const dsa_paged_cache_t* paging,
                                   const int32_t* positions, int32_t valid_len, int32_t M, int32_t H, int32_t D,
                                   int32_t S_max, float scale, uint32_t flags, float* scores, hipStream_t stream)
{
    dsa_status_t s = check_index_score(q, w, k_pool, k_scale_pool, k_dtype, M, 1, H, D, S_max, flags, scores);
    if (s != DSA_OK) return s;
    dsa::PageMap pm;
    s = check_paging(paging, S_max, &pm);
    if (s != DSA_OK) return s;
    const bool fp8 = k_dtype == DSA_KEY_FP8_E4M3;
    if (flags & DSA_SCORE_RELU)
        return launch_status(dsa::launch_score_decode_heads(q, w, k_pool, k_scale_pool, fp8, positions, valid_len, M,
                                                            H, S_max, scale, scores, nullptr, 0, &pm, stream));
    return launch_status(dsa::launch_score_decode(q, w, k_pool, k_scale_pool, fp8, positions, valid_len, M, H, S_max,
                                                  scale, scores, nullptr, 0, &pm, stream));
}

dsa_status_t dsa_sparse_attn_paged(const void* q, const void* kv_pool, const float* attn_sink,
                                   const int32_t* topk_idx, const dsa_paged_cache_t* paging, int32_t B, int32_t S,
                                   int32_t Hq, int32_t Dqk, int32_t Dv, int32_t S_kv, int32_t K_top, float sm_scale,
                                   void* out, float* lse, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream)
{
    dsa_status_t s = check_sparse_attn(q, kv_pool, topk_idx, B, S, Hq, Dqk, Dv, S_kv, K_top, out, true);
    if (s != DSA_OK) return s;
    dsa::PageMap pm;
    s = check_paging(paging, S_kv, &pm);
    if (s != DSA_OK) return s;
    const size_t need = dsa::plan::attn_partial_bytes(B, S, Hq, Dv, K_top);
    if (need > 0 && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE;
    if (need > 0 && !aligned16(workspace)) return DSA_ERR_ALIGN;
    return launch_status(dsa::launch_sparse_attn(q, kv_pool, attn_sink, topk_idx, B, S, Hq, Dqk, Dv, S_kv, K_top,
                                                 sm_scale, out, lse, workspace, &pm, stream));
}

dsa_status_t dsa_cache_write(const void* k_new, int32_t T, int32_t rows_per_seq, int32_t D,
                             const int32_t* positions, dsa_key_dtype_t k_dtype, void* k_cache, float* k_scale,
                             int32_t S_max, uint32_t flags, hipStream_t stream)
{
    const dsa_status_t s =
        check_cache_write(k_new, T, rows_per_seq, D, positions, k_dtype, k_cache, k_scale, S_max, flags);
    if (s != DSA_OK) return s;
    return launch_status(dsa::launch_cache_write(k_new, T, rows_per_seq, positions, k_dtype == DSA_KEY_FP8_E4M3,
                                                 (flags & DSA_CACHE_QDQ) != 0, (flags & DSA_CACHE_ROUND_SCALE) != 0,
                                                 k_cache, k_scale, S_max, nullptr, stream));
}

dsa_status_t dsa_cache_write_paged(const void* k_new, int32_t T, int32_t rows_per_seq, int32_t D,
                                   const int32_t* positions, dsa_key_dtype_t k_dtype, void* k_pool,
                                   float* k_scale_pool, const dsa_paged_cache_t* paging, int32_t S_max,
                                   uint32_t flags, hipStream_t stream)
{
    dsa_status_t s =
        check_cache_write(k_new, T, rows_per_seq, D, positions, k_dtype, k_pool, k_scale_pool, S_max, flags);
    if (s != DSA_OK) return s;
    dsa::PageMap pm;
    s = check_paging(paging, S_max, &pm);
    if (s != DSA_OK) return s;
    return launch_status(dsa::launch_cache_write(k_new, T, rows_per_seq, positions, k_dtype == DSA_KEY_FP8_E4M3,
                                                 (flags & DSA_CACHE_QDQ) != 0, (flags & DSA_CACHE_ROUND_SCALE) != 0,
                                                 k_pool, k_scale_pool, S_max, &pm, stream));
}

}  // extern "C"
