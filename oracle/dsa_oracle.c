/*
 * dsa_oracle.c -- plain, slow CPU oracle for the DeepSeek Sparse Attention
 * (DSA) hot path: lightning-indexer scores, top-k selection, window/top-k
 * index assembly, top-k sparse attention with an attention sink, and the
 * key-cache write with FP8 block quantisation.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and
 * the CPU-baseline leg of the benchmark may call this code.  It shares no
 * source with the HIP library (no headers, helpers, tables or constants):
 * every format decode and every formula below is written out from its
 * definition, in double precision, with no blocking, fusion or reordering.
 *
 * Sources (web pages; cited by title and section):
 *   [NKI-V32]    AWS Neuron, "DeepSeek-V3.2 Sparse Indexer Kernel API
 *                Reference" -- Parameters, Returns, Notes, Dimensions.
 *   [NKI-MX]     AWS Neuron, "Sparse Attention Indexer MX BF16Score Kernel
 *                API Reference" -- :param mask:, :return:, Notes, Dimensions.
 *   [NEMO-DSV4]  NeMo AutoModel API page
 *                "nemo_automodel.components.models.deepseek_v4.optimized_kernels"
 *                -- sparse_attention_torch, indexer_scores_torch,
 *                extract_indexer_topk_scores_torch, build_dsv4_sparse_topk_indices.
 *   [V4-KERNEL]  kwkr.cn article on the DeepSeek-V4-Pro-0813-nvfp4-DSpark
 *                inference/kernel.py -- sections on the FP8 block quantiser
 *                and on the TileLang sparse-attention kernel.
 *   [TOKAMAX]    OpenXLA tokamax "Supported Ops and Hardware", Attention
 *                Variants table -- masked_dense_mla row.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - per-head activation: identity by default (the pages only say the
 *     score is a per-head q.k weighted by per-head weights and summed);
 *     relu=1 selects max(0, .) for the published DSA variant.
 *   - accumulation precision is unstated: sums are taken in double and the
 *     score is rounded once to fp32, the output type [NKI-V32] Returns fixes.
 *   - mask bound: the most negative finite bfloat16, -0x1.FEp+127, so a
 *     bfloat16 consumer never sees -inf [NKI-V32] Notes.
 *   - the sink is a logit in the units of the scaled scores, excluded from
 *     the max; with no sink the term is absent [V4-KERNEL] sparse attention.
 *   - FP8 block quantisation: the pages fix no precision, yet its arithmetic
 *     decides integer codes, so it is done in binary32 as a GPU kernel does
 *     it: amax, scale = amax / 448, y = x / scale (each one IEEE binary32
 *     operation), y clamped to [-448, 448], then the nearest E4M3 value with
 *     ties to the even code.  An all-zero block gets scale 1.  The optional
 *     power-of-two scale is the smallest power of two >= amax / 448.
 *
 * Inputs must be free of NaN.  Threads split independent rows (or
 * (batch, query, head) triples) statically; each output element is computed
 * by exactly one thread in a fixed order, so results do not depend on the
 * thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F64 0
#define OR_BF16 1
#define OR_FP8_E4M3 2

/* -0x1.FEp+127: sign 1, exponent 254, mantissa 0x7F0000.  It is the most
 * negative finite bfloat16 (bit pattern 0xFF7F) and exact in binary32. */
static float oracle_mask_bound_value(void)
{
    uint32_t u = 0xFF7F0000u;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

float oracle_mask_bound(void) { return oracle_mask_bound_value(); }

/* bfloat16 is the upper half of an IEEE-754 binary32 word. */
static double bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP 8-bit E4M3 ("e4m3fn"): sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; exponent 0 holds subnormals m * 2^-9; no infinities; the all-ones
 * exponent and mantissa pattern is NaN; largest finite magnitude 448. */
static double fp8_e4m3_value(uint8_t c)
{
    int sign = c >> 7;
    int e = (c >> 3) & 0xF;
    int m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

void oracle_decode_bf16(const uint16_t* src, double* dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = bf16_value(src[i]);
}

void oracle_decode_fp8_e4m3(const uint8_t* src, double* dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = fp8_e4m3_value(src[i]);
}

/* Nearest E4M3 code to y (finite, |y| <= 448), found by trying every
 * non-negative finite code; of two equally near codes the even one (even
 * mantissa) wins, i.e. round to nearest, ties to even.  The sign bit is y's,
 * so a negative y that rounds to zero gives the code of -0. */
static uint8_t fp8_e4m3_encode(float y)
{
    const double v = fabs((double)y);
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        const double d = fabs(fp8_e4m3_value((uint8_t)c) - v);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best_d = d;
            best = c;
        }
    }
    return (uint8_t)(best | (signbit(y) ? 0x80 : 0));
}

void oracle_encode_fp8_e4m3(const float* src, uint8_t* dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = fp8_e4m3_encode(src[i]);
}

/* bfloat16 nearest to a finite binary32 value, ties to even (the bfloat16
 * keeps the upper 16 bits; the lower 16 decide the rounding). */
static uint16_t bf16_round(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    const uint32_t lower = u & 0xFFFFu;
    uint32_t upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;
    return (uint16_t)upper;
}

/* FP8 block quantiser, [V4-KERNEL] FP8 block quantisation (block of 128
 * elements, scale = amax / 448 so the block fits E4M3's +-448; optional
 * power-of-two scale).  x: n_blocks * block bfloat16 bit patterns; codes:
 * same count; scales: one per block.  Every step is one binary32
 * operation, see the file header. */
void oracle_quantize_fp8_blocks(const uint16_t* x, int64_t n_blocks, int32_t block, int round_scale,
                                uint8_t* codes, float* scales)
{
    for (int64_t b = 0; b < n_blocks; ++b) {
        const uint16_t* xb = x + b * block;
        float amax = 0.0f;
        for (int32_t i = 0; i < block; ++i) {
            const float a = fabsf((float)bf16_value(xb[i]));
            if (a > amax)
                amax = a;
        }
        float s = 1.0f;
        if (amax > 0.0f) {
            s = amax / 448.0f;
            if (round_scale) {
                int e;
                const float m = frexpf(s, &e); /* s = m * 2^e, m in [0.5, 1) */
                if (m != 0.5f)
                    s = ldexpf(1.0f, e);
            }
        }
        for (int32_t i = 0; i < block; ++i) {
            float y = (float)bf16_value(xb[i]) / s;
            if (y > 448.0f)
                y = 448.0f;
            if (y < -448.0f)
                y = -448.0f;
            codes[b * block + i] = fp8_e4m3_encode(y);
        }
        scales[b] = s;
    }
}

/* Dequantised bfloat16 of the codes: value(code) * scale in binary32,
 * rounded once to bfloat16 (the quantise-then-dequantise option of
 * [V4-KERNEL] FP8 block quantisation). */
void oracle_dequantize_fp8_blocks(const uint8_t* codes, const float* scales, int64_t n_blocks, int32_t block,
                                  uint16_t* out)
{
    for (int64_t b = 0; b < n_blocks; ++b)
        for (int32_t i = 0; i < block; ++i)
            out[b * block + i] = bf16_round((float)fp8_e4m3_value(codes[b * block + i]) * scales[b]);
}

/* Element i of a tensor stored as dtype (F64 / BF16 / FP8 codes). */
static double load_elem(const void* base, int dtype, int64_t i)
{
    if (dtype == OR_F64)
        return ((const double*)base)[i];
    if (dtype == OR_BF16)
        return bf16_value(((const uint16_t*)base)[i]);
    return fp8_e4m3_value(((const uint8_t*)base)[i]);
}

/* Attendable slots of row r: position+1 when positions are given (slot
 * index == absolute position), else the whole cache; an optional valid_len
 * (>= 0) caps it; the result is clamped to [0, S_max].  [NKI-V32]
 * Parameters (positions, valid_len); [NKI-MX] Dimensions (end_pos). */
int32_t oracle_n_valid(const int32_t* positions, int32_t valid_len, int64_t r, int32_t S_max)
{
    int64_t n = positions ? (int64_t)positions[r] + 1 : (int64_t)S_max;
    if (valid_len >= 0 && (int64_t)valid_len < n)
        n = valid_len;
    if (n < 0)
        n = 0;
    if (n > S_max)
        n = S_max;
    return (int32_t)n;
}

/* Lightning-indexer score [NKI-V32] Returns / Notes, [NKI-MX] :return:,
 * [NEMO-DSV4] indexer_scores_torch:
 *   score[r, s] = scale * sum_h w[r, h] * phi( sum_d q[r, h, d] * K[c, s, d] )
 * for attendable slots s < n_valid(r), with c = r / rows_per_seq the cache
 * row r reads; other slots get the finite mask bound.
 * Layouts: q [M, H, D]; w [M, H] fp32; K [M / rows_per_seq, S_max, D];
 * k_scale (FP8 keys only) [M / rows_per_seq, S_max], one scale per slot
 * (the D = 128 elements of a slot form one quantisation block). */
void oracle_index_score(const void* q, int q_dtype, const float* w, const void* k, int k_dtype,
                        const float* k_scale, const int32_t* positions, int32_t valid_len,
                        int32_t M, int32_t rows_per_seq, int32_t H, int32_t D, int32_t S_max,
                        double scale, int relu, float* scores, int nthreads)
{
    const float mask = oracle_mask_bound_value();
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
    for (int32_t r = 0; r < M; ++r) {
        const int64_t c = r / rows_per_seq;
        const int32_t nv = oracle_n_valid(positions, valid_len, r, S_max);
        for (int32_t s = 0; s < S_max; ++s) {
            if (s >= nv) {
                scores[(int64_t)r * S_max + s] = mask;
                continue;
            }
            const int64_t kbase = (c * S_max + s) * (int64_t)D;
            const double ks = (k_dtype == OR_FP8_E4M3) ? (double)k_scale[c * S_max + s] : 1.0;
            double acc = 0.0;
            for (int32_t h = 0; h < H; ++h) {
                const int64_t qbase = ((int64_t)r * H + h) * D;
                double dot = 0.0;
                for (int32_t d = 0; d < D; ++d)
                    dot += load_elem(q, q_dtype, qbase + d) * (load_elem(k, k_dtype, kbase + d) * ks);
                if (relu && dot < 0.0)
                    dot = 0.0;
                acc += (double)w[(int64_t)r * H + h] * dot;
            }
            scores[(int64_t)r * S_max + s] = (float)(scale * acc);
        }
    }
}

typedef struct {
    float score;
    int32_t slot;
} scored_slot;

/* Descending score; equal scores by ascending slot. */
static int cmp_desc(const void* a, const void* b)
{
    const scored_slot* x = (const scored_slot*)a;
    const scored_slot* y = (const scored_slot*)b;
    if (x->score > y->score)
        return -1;
    if (x->score < y->score)
        return 1;
    return (x->slot > y->slot) - (x->slot < y->slot);
}

/* Top-k [NKI-V32] Returns / Notes, [NKI-MX] :param emit_flat_topk:: per row,
 * the min(k, n_valid) highest-scoring attendable slots (a set: order carries
 * no meaning), padded with -1 to width k.  This oracle fully sorts the
 * attendable slots and lists them in sorted order; ties go to the lower
 * slot.  topk_scores (optional) gathers the selected scores, -inf where the
 * index is -1 [NEMO-DSV4] extract_indexer_topk_scores_torch. */
void oracle_topk(const float* scores, int32_t M, int32_t S_max, const int32_t* positions,
                 int32_t valid_len, int32_t k, int32_t* topk_idx, float* topk_scores, int nthreads)
{
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
    for (int32_t r = 0; r < M; ++r) {
        const int32_t nv = oracle_n_valid(positions, valid_len, r, S_max);
        scored_slot* row = (scored_slot*)malloc(sizeof(scored_slot) * (size_t)(nv > 0 ? nv : 1));
        for (int32_t s = 0; s < nv; ++s) {
            row[s].score = scores[(int64_t)r * S_max + s];
            row[s].slot = s;
        }
        qsort(row, (size_t)nv, sizeof(scored_slot), cmp_desc);
        for (int32_t j = 0; j < k; ++j) {
            const int64_t o = (int64_t)r * k + j;
            if (j < nv) {
                topk_idx[o] = row[j].slot;
                if (topk_scores)
                    topk_scores[o] = row[j].score;
            } else {
                topk_idx[o] = -1;
                if (topk_scores)
                    topk_scores[o] = -INFINITY;
            }
        }
        free(row);
    }
}

/* Index list of one decode step: the indexer's top-k plus the always-selected
 * sliding window of the last `window` attendable positions, concatenated
 * [V4-KERNEL] sparse attention (window KV always selected, concatenated with
 * the indexer's top-k); [NEMO-DSV4] build_dsv4_sparse_topk_indices.
 * Reading: the list is a set union -- a top-k entry that also lies in the
 * window is replaced by -1 so no slot is listed twice; window positions
 * below 0 are -1.  out [B, k + window]: columns [0, k) the filtered top-k,
 * columns [k, k + window) the window positions n_valid-window .. n_valid-1. */
void oracle_assemble(const int32_t* topk_idx, const int32_t* positions, int32_t valid_len,
                     int32_t B, int32_t S_max, int32_t k, int32_t window, int32_t* out)
{
    const int32_t width = k + window;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t nv = oracle_n_valid(positions, valid_len, b, S_max);
        const int32_t wstart = nv - window;
        for (int32_t j = 0; j < k; ++j) {
            const int32_t t = topk_idx[(int64_t)b * k + j];
            out[(int64_t)b * width + j] = (t < 0 || t >= wstart) ? -1 : t;
        }
        for (int32_t i = 0; i < window; ++i) {
            const int32_t p = wstart + i;
            out[(int64_t)b * width + k + i] = p < 0 ? -1 : p;
        }
    }
}

/* Top-k sparse multi-query attention with an attention sink
 * [NEMO-DSV4] sparse_attention_torch; [V4-KERNEL] sparse attention.
 * q [B, S, Hq, Dqk]; kv [B, S_kv, Dqk] (one head shared by all query heads;
 * values are its leading Dv features); sink [Hq] or NULL; idx [B, S, K_top]
 * where -1 (or any index outside [0, S_kv)) masks the entry.  Listed entries
 * count as a multiset.  For each (b, s, h), over the valid entries j:
 *   logit_j = sm_scale * q . kv[idx_j]
 *   m       = max_j logit_j
 *   l       = sum_j exp(logit_j - m) + exp(sink_h - m)   (sink term if given)
 *   out     = sum_j exp(logit_j - m) * kv[idx_j, :Dv] / l
 *   lse     = m + log(l)
 * Written as a plain two-pass softmax (not blockwise).  With no valid entry
 * the output is 0 and lse is the sink (or -inf without a sink). */
void oracle_sparse_attn(const void* q, int q_dtype, const void* kv, int kv_dtype, const float* sink,
                        const int32_t* idx, int32_t B, int32_t S, int32_t Hq, int32_t Dqk, int32_t Dv,
                        int32_t S_kv, int32_t K_top, double sm_scale, double* out, double* lse,
                        int nthreads)
{
    const int64_t n_items = (int64_t)B * S * Hq;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t item = 0; item < n_items; ++item) {
        const int32_t h = (int32_t)(item % Hq);
        const int64_t bs = item / Hq; /* b * S + s */
        const int64_t b = bs / S;
        const int32_t* ilist = idx + bs * K_top;
        double* logit = (double*)malloc(sizeof(double) * (size_t)(K_top > 0 ? K_top : 1));
        double m = -INFINITY;
        int32_t n_ok = 0;
        for (int32_t j = 0; j < K_top; ++j) {
            const int32_t t = ilist[j];
            if (t < 0 || t >= S_kv) {
                logit[j] = -INFINITY;
                continue;
            }
            double dot = 0.0;
            for (int32_t d = 0; d < Dqk; ++d)
                dot += load_elem(q, q_dtype, item * Dqk + d) *
                       load_elem(kv, kv_dtype, (b * S_kv + t) * (int64_t)Dqk + d);
            logit[j] = sm_scale * dot;
            if (logit[j] > m)
                m = logit[j];
            ++n_ok;
        }
        double* o = out + item * Dv;
        for (int32_t d = 0; d < Dv; ++d)
            o[d] = 0.0;
        if (n_ok == 0) {
            if (lse)
                lse[item] = sink ? (double)sink[h] : -INFINITY;
            free(logit);
            continue;
        }
        double l = 0.0;
        for (int32_t j = 0; j < K_top; ++j) {
            const int32_t t = ilist[j];
            if (t < 0 || t >= S_kv)
                continue;
            const double p = exp(logit[j] - m);
            l += p;
            for (int32_t d = 0; d < Dv; ++d)
                o[d] += p * load_elem(kv, kv_dtype, (b * S_kv + t) * (int64_t)Dqk + d);
        }
        if (sink)
            l += exp((double)sink[h] - m);
        for (int32_t d = 0; d < Dv; ++d)
            o[d] /= l;
        if (lse)
            lse[item] = m + log(l);
        free(logit);
    }
}

/*
 * Masked dense attention [TOKAMAX] masked_dense_mla: the attention of
 * oracle_sparse_attn over the SET of slots the list selects, written as a
 * dense pass over every slot t < S_kv of the sequence with a boolean mask.
 * mask[t] is set when some entry of the list equals t (entries that are -1
 * or outside [0, S_kv) set nothing; a slot listed twice is set once).  Then,
 * over the selected slots in slot order,
 *   m = max_t logit_t,  l = sum_t e^{logit_t - m} + e^{sink - m},
 *   out = sum_t e^{logit_t - m} kv[b, t, 0:Dv] / l,  lse = m + log l,
 * the same formula as the sparse form; no selected slot: out = 0, lse = sink.
 */
void oracle_masked_dense_attn(const void* q, int q_dtype, const void* kv, int kv_dtype, const float* sink,
                              const int32_t* idx, int32_t B, int32_t S, int32_t Hq, int32_t Dqk, int32_t Dv,
                              int32_t S_kv, int32_t K_top, double sm_scale, double* out, double* lse, int nthreads)
{
    const int64_t n_items = (int64_t)B * S * Hq;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t item = 0; item < n_items; ++item) {
        const int32_t h = (int32_t)(item % Hq);
        const int64_t bs = item / Hq; /* b * S + s */
        const int64_t b = bs / S;
        const int32_t* ilist = idx + bs * K_top;
        unsigned char* mask = (unsigned char*)calloc((size_t)S_kv, 1);
        double* logit = (double*)malloc(sizeof(double) * (size_t)S_kv);
        for (int32_t j = 0; j < K_top; ++j) {
            const int32_t t = ilist[j];
            if (t >= 0 && t < S_kv)
                mask[t] = 1;
        }
        double m = -INFINITY;
        int32_t n_sel = 0;
        for (int32_t t = 0; t < S_kv; ++t) {
            if (!mask[t])
                continue;
            double dot = 0.0;
            for (int32_t d = 0; d < Dqk; ++d)
                dot += load_elem(q, q_dtype, item * Dqk + d) *
                       load_elem(kv, kv_dtype, (b * S_kv + t) * (int64_t)Dqk + d);
            logit[t] = sm_scale * dot;
            if (logit[t] > m)
                m = logit[t];
            ++n_sel;
        }
        double* o = out + item * Dv;
        for (int32_t d = 0; d < Dv; ++d)
            o[d] = 0.0;
        if (n_sel == 0) {
            if (lse)
                lse[item] = sink ? (double)sink[h] : -INFINITY;
        } else {
            double l = 0.0;
            for (int32_t t = 0; t < S_kv; ++t) {
                if (!mask[t])
                    continue;
                const double p = exp(logit[t] - m);
                l += p;
                for (int32_t d = 0; d < Dv; ++d)
                    o[d] += p * load_elem(kv, kv_dtype, (b * S_kv + t) * (int64_t)Dqk + d);
            }
            if (sink)
                l += exp((double)sink[h] - m);
            for (int32_t d = 0; d < Dv; ++d)
                o[d] /= l;
            if (lse)
                lse[item] = m + log(l);
        }
        free(logit);
        free(mask);
    }
}
