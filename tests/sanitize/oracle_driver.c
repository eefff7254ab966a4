/* Exercises every function of the CPU oracle (oracle/dsa_oracle.c) on small
 * inputs, edge cases included, in a binary built with AddressSanitizer and
 * UndefinedBehaviorSanitizer: any out-of-bounds access, leak or undefined
 * operation aborts the run.  Values are checked only for finiteness here;
 * their correctness is pinned by the oracle tests. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

enum { F64 = 0, BF16 = 1, FP8 = 2 };

float oracle_mask_bound(void);
void oracle_decode_bf16(const uint16_t* src, double* dst, int64_t n);
void oracle_decode_fp8_e4m3(const uint8_t* src, double* dst, int64_t n);
void oracle_encode_fp8_e4m3(const float* src, uint8_t* dst, int64_t n);
void oracle_quantize_fp8_blocks(const uint16_t* x, int64_t n_blocks, int32_t block, int round_scale,
                                uint8_t* codes, float* scales);
void oracle_dequantize_fp8_blocks(const uint8_t* codes, const float* scales, int64_t n_blocks, int32_t block,
                                  uint16_t* out);
int32_t oracle_n_valid(const int32_t* positions, int32_t valid_len, int64_t r, int32_t S_max);
void oracle_index_score(const void* q, int q_dtype, const float* w, const void* k, int k_dtype,
                        const float* k_scale, const int32_t* positions, int32_t valid_len, int32_t M,
                        int32_t rows_per_seq, int32_t H, int32_t D, int32_t S_max, double scale, int relu,
                        float* scores, int nthreads);
void oracle_topk(const float* scores, int32_t M, int32_t S_max, const int32_t* positions, int32_t valid_len,
                 int32_t k, int32_t* topk_idx, float* topk_scores, int nthreads);
void oracle_assemble(const int32_t* topk_idx, const int32_t* positions, int32_t valid_len, int32_t B,
                     int32_t S_max, int32_t k, int32_t window, int32_t* out);
void oracle_sparse_attn(const void* q, int q_dtype, const void* kv, int kv_dtype, const float* sink,
                        const int32_t* idx, int32_t B, int32_t S, int32_t Hq, int32_t Dqk, int32_t Dv,
                        int32_t S_kv, int32_t K_top, double sm_scale, double* out, double* lse, int nthreads);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double uniform(void)
{
    rng = rng * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(rng >> 11) / 9007199254740992.0;
}
static uint16_t bf16_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16); /* truncation is fine for test data */
}
static void fill_bf16(uint16_t* a, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) a[i] = bf16_bits((float)(4.0 * uniform() - 2.0));
}
static int fails = 0;
static void check_finite(const char* what, const double* a, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(a[i])) {
            fprintf(stderr, "%s: non-finite value at %lld\n", what, (long long)i);
            ++fails;
            return;
        }
}

int main(void)
{
    /* format helpers: every code and a range of values */
    uint8_t codes[256];
    double vals[256];
    for (int i = 0; i < 256; ++i) codes[i] = (uint8_t)i;
    oracle_decode_fp8_e4m3(codes, vals, 256);
    uint16_t bits[512];
    double bv[512];
    for (int i = 0; i < 512; ++i) bits[i] = (uint16_t)(i * 127);
    oracle_decode_bf16(bits, bv, 512);
    float fv[1000];
    uint8_t enc[1000];
    for (int i = 0; i < 1000; ++i) fv[i] = (float)((i - 500) * 0.97);
    oracle_encode_fp8_e4m3(fv, enc, 1000);

    /* block quantiser: random, all-zero and huge blocks, both scale modes */
    enum { NB = 5, BLK = 128 };
    uint16_t x[NB * BLK], deq[NB * BLK];
    uint8_t q8[NB * BLK];
    float sc[NB];
    fill_bf16(x, NB * BLK);
    memset(x + BLK, 0, BLK * sizeof(uint16_t));
    for (int i = 0; i < BLK; ++i) x[2 * BLK + i] = bf16_bits(i % 2 ? 3.0e38f : -1.0e-30f);
    for (int rs = 0; rs < 2; ++rs) {
        oracle_quantize_fp8_blocks(x, NB, BLK, rs, q8, sc);
        oracle_dequantize_fp8_blocks(q8, sc, NB, BLK, deq);
    }

    /* indexer scores: bf16 / fp8 keys, identity / ReLU, prefill rows, positions and caps */
    enum { M = 6, H = 3, D = 128, S = 300 };
    uint16_t q[M * H * D], kb[M * S * D];
    float w[M * H], ks[M * S], scores[M * S];
    uint8_t k8[M * S * D];
    fill_bf16(q, M * H * D);
    fill_bf16(kb, M * S * D);
    for (int i = 0; i < M * H; ++i) w[i] = (float)(2.0 * uniform() - 1.0);
    for (int i = 0; i < M * S * D; ++i) k8[i] = (uint8_t)(uniform() * 256) & 0xF7; /* no NaN codes */
    for (int i = 0; i < M * S; ++i) ks[i] = (float)uniform();
    int32_t pos[M] = {-1, 0, 1, S - 2, S - 1, 5 * S};
    for (int relu = 0; relu < 2; ++relu) {
        oracle_index_score(q, BF16, w, kb, BF16, NULL, pos, -1, M, 1, H, D, S, 0.1, relu, scores, 2);
        oracle_index_score(q, BF16, w, k8, FP8, ks, NULL, 77, M, 1, H, D, S, 0.1, relu, scores, 2);
        oracle_index_score(q, BF16, w, kb, BF16, NULL, pos, 150, M, 3, H, D, S, 0.1, relu, scores, 1);
    }
    for (int i = 0; i < M * S; ++i)
        if (!isfinite(scores[i])) ++fails;

    /* top-k with k above and below n_valid, empty rows, and assembly with windows */
    int32_t idx[M * 400];
    float tsc[M * 400];
    int32_t lst[M * 600];
    oracle_index_score(q, BF16, w, kb, BF16, NULL, pos, -1, M, 1, H, D, S, 0.1, 0, scores, 2);
    const int ks_list[3] = {1, 64, 400};
    for (int a = 0; a < 3; ++a) {
        oracle_topk(scores, M, S, pos, -1, ks_list[a], idx, tsc, 2);
        oracle_topk(scores, M, S, NULL, 10, ks_list[a], idx, NULL, 1);
        oracle_assemble(idx, pos, -1, M, S, ks_list[a], 0, lst);
        oracle_assemble(idx, pos, -1, M, S, ks_list[a], 200, lst);
    }

    /* attention: masked, out-of-range and duplicate entries, with and without sink, f64 and bf16 */
    enum { B = 2, SQ = 2, HQ = 3, DQK = 64, DV = 48, SKV = 100, KT = 40 };
    uint16_t aq[B * SQ * HQ * DQK], akv[B * SKV * DQK];
    double aqd[B * SQ * HQ * DQK], out[B * SQ * HQ * DV], lse[B * SQ * HQ];
    float sink[HQ] = {0.5f, -3.0f, 20.0f};
    int32_t aidx[B * SQ * KT];
    fill_bf16(aq, B * SQ * HQ * DQK);
    fill_bf16(akv, B * SKV * DQK);
    for (int i = 0; i < B * SQ * HQ * DQK; ++i) aqd[i] = uniform() - 0.5;
    for (int i = 0; i < B * SQ * KT; ++i) {
        const double u = uniform();
        aidx[i] = u < 0.1 ? -1 : (u < 0.15 ? SKV + 3 : (int32_t)(uniform() * SKV));
    }
    for (int j = 0; j < KT; ++j) aidx[j] = -1; /* one (b, s) row fully masked */
    oracle_sparse_attn(aq, BF16, akv, BF16, sink, aidx, B, SQ, HQ, DQK, DV, SKV, KT, 0.125, out, lse, 2);
    check_finite("attention out", out, B * SQ * HQ * DV);
    oracle_sparse_attn(aqd, F64, akv, BF16, NULL, aidx, B, SQ, HQ, DQK, DV, SKV, KT, 0.125, out, NULL, 1);
    check_finite("attention out (no sink)", out, B * SQ * HQ * DV);
    (void)oracle_mask_bound();
    (void)oracle_n_valid(NULL, -1, 0, 5);
    printf("oracle driver: %s\n", fails ? "FAILED" : "ok");
    return fails ? 1 : 0;
}
