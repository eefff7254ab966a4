// Drives every C entry point of libdsa's host side (dsa_api.cpp, linked
// with host stand-ins for the launchers) through valid and invalid
// arguments in a binary built with AddressSanitizer and
// UndefinedBehaviorSanitizer.  Device pointers are fake, aligned addresses
// that nothing dereferences.  Decode-step argument structs are allocated
// with exactly their declared struct_size, so a read past the fields a
// caller's struct holds is reported as a heap overflow.
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "dsa.h"

extern int g_launches;

static int fails = 0;
#define EXPECT(call, want)                                                                          \
    do {                                                                                            \
        const dsa_status_t got_ = (call);                                                           \
        if (got_ != (want)) {                                                                       \
            std::fprintf(stderr, "line %d: %s -> %d, expected %d\n", __LINE__, #call, got_, want); \
            ++fails;                                                                                \
        }                                                                                           \
    } while (0)

static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }
static const uintptr_t A = 0x10000;

static dsa_decode_args_t* decode_args(size_t struct_size)
{
    dsa_decode_args_t full{};
    full.struct_size = struct_size;
    full.index_q = P(A); full.index_w = static_cast<const float*>(P(A)); full.k_cache = P(A);
    full.q = P(A); full.kv = P(A); full.out = P(A);
    full.B = 4; full.H = 64; full.S_max = 65536; full.valid_len = -1; full.index_scale = 0.1f;
    full.index_topk = 1024; full.window = 128; full.Hq = 128; full.Dqk = 576; full.Dv = 512; full.sm_scale = 0.04f;
    auto* a = static_cast<dsa_decode_args_t*>(std::malloc(struct_size));
    std::memcpy(a, &full, struct_size);
    return a;
}

int main()
{
    std::printf("%s %s %g\n", dsa_version(), dsa_status_string(DSA_ERR_SHAPE), (double)dsa_mask_bound());
    for (int s = -1; s <= 7; ++s) (void)dsa_status_string(static_cast<dsa_status_t>(s));
    const float* f = static_cast<const float*>(P(A));
    float* fo = static_cast<float*>(P(A));

    // index score
    EXPECT(dsa_index_score(P(A), f, P(A), nullptr, DSA_KEY_BF16, nullptr, -1, 16, 1, 64, 128, 32768, 0.1f, 0, fo,
                           nullptr), DSA_OK);
    EXPECT(dsa_index_score(nullptr, f, P(A), nullptr, DSA_KEY_BF16, nullptr, -1, 16, 1, 64, 128, 32768, 0.1f, 0, fo,
                           nullptr), DSA_ERR_NULL);
    EXPECT(dsa_index_score(P(A), f, P(A), nullptr, DSA_KEY_BF16, nullptr, -1, 16, 1, 64, 64, 32768, 0.1f, 0, fo,
                           nullptr), DSA_ERR_UNSUPPORTED);
    EXPECT(dsa_index_score(P(A), f, P(A), nullptr, DSA_KEY_BF16, nullptr, -1, 16, 1, 65, 128, 32768, 0.1f,
                           DSA_SCORE_RELU, fo, nullptr), DSA_ERR_UNSUPPORTED);
    EXPECT(dsa_index_score(P(A), f, P(A), nullptr, DSA_KEY_FP8_E4M3, nullptr, -1, 16, 1, 64, 128, 32768, 0.1f, 0,
                           fo, nullptr), DSA_ERR_NULL);
    EXPECT(dsa_index_score(P(A), f, P(A), nullptr, DSA_KEY_BF16, nullptr, -1, 8192, 8192, 64, 128, 8192, 0.1f, 0,
                           fo, nullptr), DSA_OK);
    EXPECT(dsa_index_score(P(A), f, P(A), nullptr, DSA_KEY_BF16, nullptr, -1, 8192, 8192, 64, 128, INT32_MAX, 0.1f,
                           0, fo, nullptr), DSA_ERR_SHAPE);
    EXPECT(dsa_index_score(P(A + 4), f, P(A), nullptr, DSA_KEY_BF16, nullptr, -1, 1, 1, 4, 128, 100, 0.1f, 0, fo,
                           nullptr), DSA_ERR_ALIGN);
    EXPECT(dsa_index_score(P(A), f, P(A), nullptr, static_cast<dsa_key_dtype_t>(7), nullptr, -1, 1, 1, 4, 128, 100,
                           0.1f, 0, fo, nullptr), DSA_ERR_UNSUPPORTED);

    // top-k
    int32_t* io = static_cast<int32_t*>(P(A));
    const size_t tws = dsa_topk_workspace_size(64, 65536, 1024);
    EXPECT(dsa_topk(f, 64, 65536, nullptr, -1, 1024, io, nullptr, P(A), tws, nullptr), DSA_OK);
    EXPECT(dsa_topk(f, 64, 65536, nullptr, -1, 1024, io, nullptr, P(A), tws - 1, nullptr), DSA_ERR_WORKSPACE);
    EXPECT(dsa_topk(f, 64, DSA_MAX_TOPK_SLOTS + 1, nullptr, -1, 1024, io, nullptr, P(A), SIZE_MAX, nullptr),
           DSA_ERR_SHAPE);
    EXPECT(dsa_topk(f, 64, 65536, nullptr, -1, DSA_MAX_TOPK + 1, io, nullptr, P(A), tws, nullptr),
           DSA_ERR_UNSUPPORTED);
    EXPECT(dsa_topk(f, INT32_MAX, INT32_MAX, nullptr, -1, 1, io, nullptr, nullptr, 0, nullptr), DSA_ERR_SHAPE);
    (void)dsa_topk_workspace_size(INT32_MAX, DSA_MAX_TOPK_SLOTS, 1);
    (void)dsa_topk_workspace_size(-1, -1, -1);

    // sparse attention (contiguous and paged)
    const size_t aws = dsa_sparse_attn_workspace_size(2, 1, 128, 512, 1152);
    EXPECT(dsa_sparse_attn(P(A), P(A), f, io, 2, 1, 128, 576, 512, 65536, 1152, 0.04f, P(A), fo, P(A), aws, nullptr),
           DSA_OK);
    EXPECT(dsa_sparse_attn(P(A), P(A), f, io, 2, 1, 128, 576, 528, 65536, 1152, 0.04f, P(A), fo, P(A), aws,
                           nullptr), DSA_ERR_UNSUPPORTED);
    EXPECT(dsa_sparse_attn(P(A), P(A), f, io, 2, 1, 128, 576, 512, INT32_MAX, 1152, 0.04f, P(A), fo, P(A), aws,
                           nullptr), DSA_ERR_SHAPE);
    EXPECT(dsa_sparse_attn(P(A), P(A), f, io, 70000, 1, 128, 576, 512, 100, 1152, 0.04f, P(A), fo, P(A), aws,
                           nullptr), DSA_ERR_SHAPE);
    (void)dsa_sparse_attn_workspace_size(INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX);
    // masked-dense attention: the workspace holds every token's dense slot list, then the partials
    const size_t mws = dsa_sparse_attn_masked_dense_workspace_size(2, 1, 128, 512, 4096);
    EXPECT(mws >= 2u * 4096u * 4u ? DSA_OK : DSA_ERR_SHAPE, DSA_OK);
    EXPECT(dsa_sparse_attn_masked_dense(P(A), P(A), f, io, 2, 1, 128, 576, 512, 4096, 1152, 0.04f, P(A), fo, P(A),
                                        mws, nullptr), DSA_OK);
    EXPECT(dsa_sparse_attn_masked_dense(P(A), P(A), f, io, 2, 1, 128, 576, 512, 4096, 1152, 0.04f, P(A), fo, P(A),
                                        mws - 1, nullptr), DSA_ERR_WORKSPACE);
    EXPECT(dsa_sparse_attn_masked_dense(P(A), P(A), f, io, 2, 1, 128, 576, 512, 4096, 1152, 0.04f, P(A), fo,
                                        nullptr, 0, nullptr), DSA_ERR_WORKSPACE);
    EXPECT(dsa_sparse_attn_masked_dense(P(A), P(A), f, io, 2, 1, 128, 576, 512, DSA_MASKED_DENSE_MAX_SLOTS + 1, 64,
                                        0.04f, P(A), fo, P(A), mws, nullptr), DSA_ERR_SHAPE);
    EXPECT(dsa_sparse_attn_masked_dense(P(A), P(A), f, io, 2, 1, 128, 576, 528, 4096, 64, 0.04f, P(A), fo, P(A), mws,
                                        nullptr), DSA_ERR_UNSUPPORTED);
    EXPECT(dsa_sparse_attn_masked_dense(P(A), P(A), f, io, 2, 1, 128, 576, 512, 4096, 64, 0.04f, P(A), fo, P(A + 8),
                                        mws, nullptr), DSA_ERR_ALIGN);
    EXPECT(dsa_sparse_attn_masked_dense_workspace_size(2, 1, 128, 512, DSA_MASKED_DENSE_MAX_SLOTS + 1) == 0
               ? DSA_OK : DSA_ERR_SHAPE, DSA_OK);
    (void)dsa_sparse_attn_masked_dense_workspace_size(INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX);
    (void)dsa_sparse_attn_masked_dense_workspace_size(65535, 1, DSA_MAX_ATTN_HEADS, 512, DSA_MASKED_DENSE_MAX_SLOTS);
    int32_t table_storage[4] = {0, 1, 2, 3};
    dsa_paged_cache_t pg{table_storage, 4, 64, 4};
    EXPECT(dsa_sparse_attn_paged(P(A), P(A), f, io, &pg, 2, 1, 16, 192, 128, 256, 64, 0.07f, P(A), fo, P(A), 0,
                                 nullptr), DSA_OK);
    pg.page_size = 96;
    EXPECT(dsa_sparse_attn_paged(P(A), P(A), f, io, &pg, 2, 1, 16, 192, 128, 256, 64, 0.07f, P(A), fo, P(A), 0,
                                 nullptr), DSA_ERR_UNSUPPORTED);
    pg.page_size = 64;
    pg.n_pages = INT32_MAX;
    EXPECT(dsa_index_score_paged(P(A), f, P(A), nullptr, DSA_KEY_BF16, &pg, nullptr, -1, 2, 4, 128, 256, 0.1f, 0, fo,
                                 nullptr), DSA_ERR_SHAPE);
    pg.n_pages = 4;
    EXPECT(dsa_index_score_paged(P(A), f, P(A), nullptr, DSA_KEY_BF16, &pg, nullptr, -1, 2, 4, 128, 256, 0.1f, 0, fo,
                                 nullptr), DSA_OK);

    // decode step: full-size struct, and structs that end before the later fields
    const size_t sizes[3] = {sizeof(dsa_decode_args_t), offsetof(dsa_decode_args_t, paging),
                             offsetof(dsa_decode_args_t, index_flags)};
    for (size_t sz : sizes) {
        dsa_decode_args_t* a = decode_args(sz);
        const size_t ws = dsa_decode_step_workspace_size(a);
        EXPECT(dsa_decode_step(a, P(A), ws, nullptr), DSA_OK);
        EXPECT(dsa_decode_step(a, nullptr, 0, nullptr), DSA_ERR_WORKSPACE);
        a->Dv = 528;
        EXPECT(dsa_decode_step(a, P(A), ws, nullptr), DSA_ERR_UNSUPPORTED);
        a->Dv = 512;
        a->S_max = DSA_MAX_TOPK_SLOTS + 1;
        EXPECT(dsa_decode_step(a, P(A), SIZE_MAX, nullptr), DSA_ERR_SHAPE);
        std::free(a);
    }
    dsa_decode_args_t* small = decode_args(8);
    EXPECT(dsa_decode_step(small, P(A), 1 << 30, nullptr), DSA_ERR_UNSUPPORTED);
    (void)dsa_decode_step_workspace_size(small);
    std::free(small);
    EXPECT(dsa_decode_step(nullptr, nullptr, 0, nullptr), DSA_ERR_NULL);

    // cache write
    EXPECT(dsa_cache_write(P(A), 4, 1, 128, io, DSA_KEY_FP8_E4M3, P(A), fo, 100, DSA_CACHE_ROUND_SCALE, nullptr),
           DSA_OK);
    EXPECT(dsa_cache_write(nullptr, 0, 1, 128, nullptr, DSA_KEY_BF16, P(A), nullptr, 100, 0, nullptr), DSA_OK);
    EXPECT(dsa_cache_write(P(A), 4, 3, 128, io, DSA_KEY_BF16, P(A), nullptr, 100, 0, nullptr), DSA_ERR_SHAPE);
    EXPECT(dsa_cache_write(P(A), 4, 1, 128, io, DSA_KEY_FP8_E4M3, P(A), fo, 100, DSA_CACHE_QDQ, nullptr),
           DSA_ERR_UNSUPPORTED);
    EXPECT(dsa_cache_write_paged(P(A), 4, 1, 128, io, DSA_KEY_BF16, P(A), nullptr, &pg, 256, 0, nullptr), DSA_OK);

    std::printf("api driver: %d launches, %s\n", g_launches, fails ? "FAILED" : "ok");
    return fails ? 1 : 0;
}
