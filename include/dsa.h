/*
 * dsa.h -- C ABI of libdsa, the MI355X (gfx950) implementation of the
 * DeepSeek Sparse Attention (DSA) hot path:
 *
 *   dsa_index_score   lightning-indexer score of every cached key slot
 *   dsa_topk          the index_topk best attendable slots (unordered set)
 *   dsa_sparse_attn   top-k sparse multi-query attention with attention sink
 *   dsa_decode_step   the three fused into one decode step on one stream,
 *                     with the always-selected sliding window
 *   dsa_cache_write   new keys stored in the key cache at their positions,
 *                     optionally FP8 block-quantised
 *   dsa_sparse_attn_masked_dense
 *                     the same attention over the set of listed slots,
 *                     computed densely over a short sequence
 *   dsa_index_score_paged, dsa_sparse_attn_paged, dsa_cache_write_paged
 *                     the decode scorer, the attention and the key write
 *                     over paged caches (a block table into a page pool)
 *
 * Sources (web pages, cited by title and section):
 *   [NKI-V32]   AWS Neuron "DeepSeek-V3.2 Sparse Indexer Kernel API Reference"
 *   [NKI-MX]    AWS Neuron "Sparse Attention Indexer MX BF16Score Kernel API Reference"
 *   [NEMO-DSV4] NeMo AutoModel API page
 *               "nemo_automodel.components.models.deepseek_v4.optimized_kernels"
 *   [V4-KERNEL] kwkr.cn article on DeepSeek-V4-Pro-0813-nvfp4-DSpark
 *               inference/kernel.py (sparse-attention and FP8 sections)
 *   [TOKAMAX]   OpenXLA tokamax "Supported Ops and Hardware", Attention
 *               Variants table (lightning_indexer, batched_rpa,
 *               masked_dense_mla rows)
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE memory on the current HIP device, owned by
 *     the caller, dense row-major in the layout stated, 16-byte aligned.
 *     The library never allocates, frees or keeps a pointer; scratch space
 *     is the caller's `workspace` (size from the matching *_workspace_size
 *     query, which needs no GPU).  The one exception is
 *     dsa_decode_step_static, whose scratch is a library-owned device array.
 *   - All work is enqueued on `stream` (NULL = the default stream); no call
 *     synchronises the host.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     any error status no output has been touched.  DSA_ERR_LAUNCH reports a
 *     launch failure; faults during execution surface at the caller's next
 *     synchronisation.  No C++ exception crosses this interface.  Calls are
 *     thread-safe; the library holds no state beyond the scratch array of
 *     dsa_decode_step_static and its device address per GPU.
 *   - bf16 = bfloat16; fp8 = OCP FP8 E4M3 ("e4m3fn", max 448) bytes.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status {
    DSA_OK = 0,
    DSA_ERR_NULL = 1,        /* a required pointer is NULL */
    DSA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
    DSA_ERR_UNSUPPORTED = 3, /* valid request this build does not implement */
    DSA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
    DSA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
    DSA_ERR_LAUNCH = 6       /* a kernel launch failed (hipGetLastError) */
} dsa_status_t;

typedef enum dsa_key_dtype {
    DSA_KEY_BF16 = 0,     /* key cache in bfloat16 */
    DSA_KEY_FP8_E4M3 = 1  /* OCP FP8 E4M3 codes + one fp32 scale per slot */
} dsa_key_dtype_t;

/* flags of dsa_index_score */
#define DSA_SCORE_RELU 1u /* per-head activation max(0, .) before weighting */

#define DSA_INDEX_HEAD_DIM 128 /* indexer head_dim: [NKI-V32] Dimensions; [NKI-MX] usage */
#define DSA_MAX_TOPK 2048
#define DSA_MAX_TOPK_SLOTS (1 << 24) /* slots per row of dsa_topk / dsa_decode_step */
#define DSA_MAX_ATTN_DIM 576
#define DSA_MAX_ATTN_VDIM 512 /* value features: the output accumulator holds 32 heads x 512 per wave */
#define DSA_MAX_ATTN_HEADS 65535 /* query heads of the attention (keeps launch grids in range) */
#define DSA_MASKED_DENSE_MAX_SLOTS 65536 /* sequence length of dsa_sparse_attn_masked_dense */

/* Library version string, e.g. "0.1.0". */
const char* dsa_version(void);

/* Human-readable name of a status code (static storage). */
const char* dsa_status_string(dsa_status_t status);

/* The finite mask bound written for slots a row cannot attend to:
 * -0x1.FEp+127f, the most negative finite bfloat16, exact in fp32.  A finite
 * bound (not -inf) keeps a bfloat16 consumer's max-select NaN-free
 * [NKI-V32] Notes. */
float dsa_mask_bound(void);

/*
 * dsa_index_score -- lightning-indexer scores [NKI-V32] Returns and Notes;
 * [NKI-MX] :return: and Dimensions; [NEMO-DSV4] indexer_scores_torch.
 * (The pages name no activation; the published DSA indexer applies ReLU per
 * head, hence the flag.)
 *
 *   scores[r, s] = scale * sum_h w[r, h] * phi( sum_d q[r, h, d] * K[c, s, d] )
 *
 * for every slot s < n_valid(r), where c = r / rows_per_seq is the cache row
 * r reads and phi is the identity (flags = 0) or max(0, .) (DSA_SCORE_RELU).
 * Slots s >= n_valid(r) get dsa_mask_bound() exactly.
 *
 * n_valid(r) = positions[r] + 1 if positions != NULL, else S_max; capped by
 * valid_len when valid_len >= 0; clamped to [0, S_max] ([NKI-V32]
 * Parameters positions / valid_len).  Decode: one row per sequence
 * (rows_per_seq = 1).  Prefill: rows_per_seq query rows share one cache and
 * positions[r] = start_pos + (r mod rows_per_seq) gives the causal range
 * ([NKI-MX] Dimensions: end_pos = start_pos + S).
 *
 *   q        [M, H, D] bf16, device
 *   w        [M, H] fp32 per-head weights, device
 *   k_cache  [M / rows_per_seq, S_max, D] bf16, or fp8 E4M3 bytes, device
 *   k_scale  [M / rows_per_seq, S_max] fp32, one scale per slot (fp8 only;
 *            must be NULL for bf16)
 *   positions [M] int32 or NULL, device
 *   scores   [M, S_max] fp32 output, device
 *
 * Limits: D == 128; 1 <= H <= 128; M >= 1; S_max >= 1; M % rows_per_seq == 0.
 * rows_per_seq == 1: M <= 65535; with DSA_SCORE_RELU also H <= 64.
 * rows_per_seq > 1 requires bf16 keys and S_max * 256 bytes below 2 GiB, and
 * with DSA_SCORE_RELU also H <= 64.  (With the identity activation the
 * heads fold by linearity into one fp32 query per row, as in decode.)
 * Otherwise DSA_ERR_SHAPE / DSA_ERR_UNSUPPORTED.
 */
dsa_status_t dsa_index_score(const void* q, const float* w, const void* k_cache, const float* k_scale,
                             dsa_key_dtype_t k_dtype, const int32_t* positions, int32_t valid_len,
                             int32_t M, int32_t rows_per_seq, int32_t H, int32_t D, int32_t S_max,
                             float scale, uint32_t flags, float* scores, hipStream_t stream);

/*
 * dsa_topk -- per row, the min(index_topk, n_valid(r)) highest-scoring
 * attendable slots, padded with -1 to width index_topk.  The row is an
 * unordered set: column order carries no meaning ([NKI-V32] Returns and
 * Notes; [NKI-MX] :param emit_flat_topk:).  Among equal scores at the
 * selection boundary any subset of the right size may be returned.
 *
 *   scores      [M, S_max] fp32, device (NaN-free)
 *   positions / valid_len: as dsa_index_score (rows_per_seq = 1 rule)
 *   topk_idx    [M, index_topk] int32 output, device
 *   topk_scores [M, index_topk] fp32 output or NULL: the selected scores,
 *               -inf where the index is -1 ([NEMO-DSV4]
 *               extract_indexer_topk_scores_torch)
 *
 * The output is deterministic: the same scores give the same row, column
 * for column, on every call (ties at the boundary included).
 *
 * Limits: 1 <= index_topk <= DSA_MAX_TOPK; M >= 1;
 * 1 <= S_max <= DSA_MAX_TOPK_SLOTS.  The workspace (size from
 * dsa_topk_workspace_size; 0 for many short rows) must be 16-byte aligned
 * (DSA_ERR_ALIGN otherwise); its contents on entry do not matter.
 */
size_t dsa_topk_workspace_size(int32_t M, int32_t S_max, int32_t index_topk);
dsa_status_t dsa_topk(const float* scores, int32_t M, int32_t S_max, const int32_t* positions,
                      int32_t valid_len, int32_t index_topk, int32_t* topk_idx, float* topk_scores,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dsa_sparse_attn -- top-k sparse multi-query attention with a learnable
 * sink ([NEMO-DSV4] sparse_attention_torch; [V4-KERNEL] sparse-attention
 * section).  For each batch b, query s and head h, over the listed entries
 * j with 0 <= topk_idx[b, s, j] < S_kv (others, including -1, are masked and
 * never read; listed entries count as a multiset):
 *
 *   logit_j = sm_scale * q[b, s, h, :] . kv[b, idx_j, :]
 *   out     = sum_j e^{logit_j - m} kv[b, idx_j, 0:Dv]
 *             / (sum_j e^{logit_j - m} + e^{attn_sink[h] - m}),  m = max_j logit_j
 *   lse     = m + log(denominator)
 *
 * The sink is a logit in the units of the scaled scores; attn_sink = NULL
 * removes the term.  With no valid entry, out = 0 and lse = attn_sink[h]
 * (or -inf).
 *
 *   q         [B, S, Hq, Dqk] bf16, device
 *   kv        [B, S_kv, Dqk] bf16, device (single head shared by all query
 *             heads; the value is its leading Dv features)
 *   attn_sink [Hq] fp32 or NULL, device
 *   topk_idx  [B, S, K_top] int32, device
 *   out       [B, S, Hq, Dv] bf16 output, device
 *   lse       [B, S, Hq] fp32 output or NULL, device
 *
 * Limits: Dqk % 32 == 0, 32 <= Dqk <= 576; Dv % 16 == 0, 16 <= Dv <= min(Dqk, 512);
 * B, S, K_top >= 1; 1 <= Hq <= DSA_MAX_ATTN_HEADS; S_kv >= 1; B * S <= 65535;
 * one sequence's KV (S_kv * Dqk * 2 bytes) below 2 GiB.  The workspace
 * (size from dsa_sparse_attn_workspace_size; 0 when there are enough query
 * tokens to fill the GPU, and for shapes the call rejects) holds per-split
 * partial results when few tokens are given; it must be 16-byte aligned.
 */
size_t dsa_sparse_attn_workspace_size(int32_t B, int32_t S, int32_t Hq, int32_t Dv, int32_t K_top);
dsa_status_t dsa_sparse_attn(const void* q, const void* kv, const float* attn_sink, const int32_t* topk_idx,
                             int32_t B, int32_t S, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t S_kv,
                             int32_t K_top, float sm_scale, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * dsa_sparse_attn_masked_dense -- the attention of dsa_sparse_attn over the
 * SET of slots topk_idx lists, computed densely: every slot p < S_kv of the
 * sequence enters the softmax in slot order and is masked unless listed
 * ([TOKAMAX] masked_dense_mla row: latent attention restricted to a selected
 * top-k subset through a dense mask, for shorter sequences).  Entries that
 * are -1 or outside [0, S_kv) select nothing; a slot listed more than once
 * counts once (dsa_sparse_attn counts every entry, so the two agree on
 * lists without repeats, such as dsa_topk's).  q, kv, attn_sink, out, lse
 * and the formulas are those of dsa_sparse_attn, with j running over the
 * selected slots.
 *
 * The work grows with S_kv (all slots are read and scored), not with K_top:
 * the form pays when the selection covers much of a short sequence.
 *
 * Limits: as dsa_sparse_attn, and S_kv <= DSA_MASKED_DENSE_MAX_SLOTS.  The
 * workspace (always needed; size from
 * dsa_sparse_attn_masked_dense_workspace_size, 0 for shapes the call
 * rejects) holds the dense mask of every query token as a slot list
 * (B * S * S_kv int32) and the attention's partial results; it must be
 * 16-byte aligned.
 */
size_t dsa_sparse_attn_masked_dense_workspace_size(int32_t B, int32_t S, int32_t Hq, int32_t Dv, int32_t S_kv);
dsa_status_t dsa_sparse_attn_masked_dense(const void* q, const void* kv, const float* attn_sink,
                                          const int32_t* topk_idx, int32_t B, int32_t S, int32_t Hq, int32_t Dqk,
                                          int32_t Dv, int32_t S_kv, int32_t K_top, float sm_scale, void* out,
                                          float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Paged caches ([TOKAMAX] lightning_indexer scores over a paged KV cache;
 * batched_rpa attends over one).  A sequence's slots are cut into runs of
 * page_size consecutive slots; run p of sequence r lives in page
 * block_table[r * max_pages + p] of a pool shared by all sequences, so
 * slot s of sequence r is pool row
 *   block_table[r * max_pages + s / page_size] * page_size + s % page_size.
 * Pools: keys [n_pages * page_size, 128] (bf16, or fp8 codes with scales
 * [n_pages * page_size] fp32), KV [n_pages * page_size, Dqk] bf16.
 * Table entries for slots a call reads must lie in [0, n_pages); an entry
 * outside it is clamped into the pool (wrong data, no fault).
 *
 * Limits: page_size a power of two, 64 <= page_size <= 65536;
 * max_pages >= 1; n_pages >= 1; n_pages * page_size < 2^31; the logical
 * slot range (S_max, S_kv) at most max_pages * page_size.
 */
typedef struct dsa_paged_cache {
    const int32_t* block_table; /* [n_seq, max_pages] int32, device */
    int32_t max_pages;          /* columns of block_table */
    int32_t page_size;          /* slots per page */
    int32_t n_pages;            /* pages in the pool */
} dsa_paged_cache_t;

/*
 * dsa_decode_step -- one DSA decode step for B sequences (one query token
 * each): indexer score of every cached slot -> top-k -> index list =
 * top-k plus the always-selected window of the last `window` attendable
 * positions (a set union: top-k entries inside the window become -1;
 * window positions below 0 are -1) -> sparse attention over that list
 * ([V4-KERNEL] sparse-attention section, use in Attention.forward;
 * [NEMO-DSV4] build_dsv4_sparse_topk_indices).  The key cache slot s and
 * the kv slot s are the same position, so S_kv == S_max.
 *
 * The struct is versioned by struct_size (set it to sizeof(dsa_decode_args_t));
 * fields added later read as 0 / NULL when struct_size ends before them
 * (the oldest accepted size ends before index_flags).
 *
 * With paging != NULL, k_cache / k_scale and kv are page pools (see
 * dsa_paged_cache_t) sharing one block table, and S_max is the logical slot
 * count of every sequence.
 *
 * Every stage is deterministic (the index list included, column for
 * column), so the same inputs give bitwise-identical outputs on every call.
 * Limits: those of the three stages; B <= 65535; S_max <= DSA_MAX_TOPK_SLOTS.
 */
typedef struct dsa_decode_args {
    size_t struct_size;
    /* indexer */
    const void* index_q;        /* [B, H, 128] bf16 */
    const float* index_w;       /* [B, H] fp32 */
    const void* k_cache;        /* [B, S_max, 128] bf16 or fp8 */
    const float* k_scale;       /* [B, S_max] fp32 (fp8 only) or NULL */
    dsa_key_dtype_t k_dtype;
    const int32_t* positions;   /* [B] int32 or NULL */
    int32_t valid_len;          /* < 0: none */
    int32_t B, H, S_max;
    float index_scale;
    int32_t index_topk;         /* 1 .. DSA_MAX_TOPK */
    int32_t window;             /* >= 0 */
    /* attention */
    const void* q;              /* [B, 1, Hq, Dqk] bf16 */
    const void* kv;             /* [B, S_max, Dqk] bf16 */
    const float* attn_sink;     /* [Hq] fp32 or NULL */
    int32_t Hq, Dqk, Dv;
    float sm_scale;
    /* outputs */
    void* out;                  /* [B, 1, Hq, Dv] bf16 */
    float* lse;                 /* [B, 1, Hq] fp32 or NULL */
    float* scores;              /* [B, S_max] fp32 or NULL (then kept in workspace) */
    int32_t* index_list;        /* [B, index_topk + window] int32 or NULL (then workspace) */
    /* added later; a struct_size that ends before this field reads as 0 */
    uint32_t index_flags;       /* flags of dsa_index_score (DSA_SCORE_RELU: H <= 64) */
    const dsa_paged_cache_t* paging; /* NULL: contiguous caches */
} dsa_decode_args_t;

size_t dsa_decode_step_workspace_size(const dsa_decode_args_t* args);
dsa_status_t dsa_decode_step(const dsa_decode_args_t* args, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * dsa_decode_step_static -- dsa_decode_step for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, kernels and
 * results as dsa_decode_step, but the step's scratch space is a
 * library-owned device array of DSA_STATIC_SCRATCH_BYTES instead of a
 * caller workspace; the caller still provides every input and output.
 *
 * The array exists once per GPU (the current device at the call), from the
 * first call on that GPU until the process ends; the call allocates nothing
 * and calls no allocating routine.  Every call on one GPU shares that GPU's
 * array: calls that may overlap on one GPU (different streams, or different
 * host threads without ordering) race and must be serialised by the caller.
 * Contents left by an earlier call are never read.
 *
 * Errors: as dsa_decode_step for invalid arguments; DSA_ERR_WORKSPACE when
 * dsa_decode_step_workspace_size(args) exceeds DSA_STATIC_SCRATCH_BYTES
 * (pass scores / index_list outputs to shrink it); DSA_ERR_LAUNCH when the
 * array's device address cannot be obtained or a launch fails.
 */
#define DSA_STATIC_SCRATCH_BYTES ((size_t)128 << 20) /* 128 MiB per GPU */
dsa_status_t dsa_decode_step_static(const dsa_decode_args_t* args, hipStream_t stream);


/* dsa_index_score over a paged key cache, one query row per sequence
 * (rows_per_seq = 1); arguments and results as dsa_index_score, with
 * k_cache / k_scale the page pools and S_max the logical slot count of
 * every sequence (the width of scores). */
dsa_status_t dsa_index_score_paged(const void* q, const float* w, const void* k_pool, const float* k_scale_pool,
                                   dsa_key_dtype_t k_dtype, const dsa_paged_cache_t* paging,
                                   const int32_t* positions, int32_t valid_len, int32_t M, int32_t H, int32_t D,
                                   int32_t S_max, float scale, uint32_t flags, float* scores, hipStream_t stream);

/* dsa_sparse_attn over a paged KV pool: topk_idx holds logical slots of
 * each sequence (masked unless 0 <= slot < S_kv), looked up through the
 * block table; the pool has no size limit beyond the page limits below.  Workspace as for
 * dsa_sparse_attn (same size query). */
dsa_status_t dsa_sparse_attn_paged(const void* q, const void* kv_pool, const float* attn_sink,
                                   const int32_t* topk_idx, const dsa_paged_cache_t* paging, int32_t B, int32_t S,
                                   int32_t Hq, int32_t Dqk, int32_t Dv, int32_t S_kv, int32_t K_top, float sm_scale,
                                   void* out, float* lse, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* flags of dsa_cache_write */
#define DSA_CACHE_ROUND_SCALE 1u /* power-of-two scale: the smallest 2^e >= amax / 448 */
#define DSA_CACHE_QDQ 2u         /* bf16 cache: store the key quantised and dequantised again */

/*
 * dsa_cache_write -- store each token's new indexer key in the key cache,
 * in place at the token's position ([NKI-V32] key_cache), optionally
 * quantised to FP8 with one scale per 128-element block ([V4-KERNEL] FP8
 * block quantisation: scale = amax / 448 so the block fits E4M3's +-448;
 * optional power-of-two scale; optional quantise-then-dequantise).
 *
 * Token t (0 <= t < T) goes to cache row c = t / rows_per_seq, slot
 * p = positions[t]; a token whose p is outside [0, S_max) is skipped.  Two
 * tokens of one row with the same position race (either may win).
 *   DSA_KEY_FP8_E4M3: amax = max_d |k[t, d]|; s = amax / 448 (1 when
 *     amax == 0), with DSA_CACHE_ROUND_SCALE the smallest power of two >= that;
 *     code[d] = the E4M3 value nearest to clamp(k[t, d] / s, -448, 448), ties
 *     to the even code (a negative value that rounds to zero gives -0); each
 *     step is one binary32 operation, so the codes equal those of any exact
 *     binary32 evaluation.  k_scale[c, p] = s.
 *   DSA_KEY_BF16: the key as given; with DSA_CACHE_QDQ the bfloat16 nearest
 *     to value(code[d]) * s (binary32 product) instead.
 *
 *   k_new     [T, 128] bf16, device
 *   positions [T] int32, device
 *   k_cache   [T / rows_per_seq, S_max, 128] bf16 or fp8 bytes, device, updated in place
 *   k_scale   [T / rows_per_seq, S_max] fp32, device (fp8 only; must be NULL for bf16)
 *
 * Limits: D == 128; T >= 0 (T == 0 enqueues nothing, and k_new and
 * positions may then be NULL); rows_per_seq >= 1 and
 * T % rows_per_seq == 0; S_max >= 1; DSA_CACHE_QDQ only with a bf16 cache;
 * DSA_CACHE_ROUND_SCALE only where a scale is computed (fp8, or bf16 with
 * DSA_CACHE_QDQ).  k_new must not overlap the cache.  Inputs must be
 * finite.
 */
dsa_status_t dsa_cache_write(const void* k_new, int32_t T, int32_t rows_per_seq, int32_t D,
                             const int32_t* positions, dsa_key_dtype_t k_dtype, void* k_cache, float* k_scale,
                             int32_t S_max, uint32_t flags, hipStream_t stream);

/* dsa_cache_write into paged caches (see dsa_paged_cache_t): token t's key
 * goes to pool row block_table[c][p / page_size] * page_size + p % page_size
 * of k_pool (and its scale to the same row of k_scale_pool), c = t /
 * rows_per_seq, p = positions[t]; positions outside [0, S_max) are skipped;
 * S_max (the logical slot count) at most max_pages * page_size. */
dsa_status_t dsa_cache_write_paged(const void* k_new, int32_t T, int32_t rows_per_seq, int32_t D,
                                   const int32_t* positions, dsa_key_dtype_t k_dtype, void* k_pool,
                                   float* k_scale_pool, const dsa_paged_cache_t* paging, int32_t S_max,
                                   uint32_t flags, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
