// Host-side launch planning of libdsa: which kernel path a call takes and
// how much workspace it needs.  Plain C++ (no device code), shared by the
// kernels' launchers and the C entry points, and small enough to build on
// its own with the host sanitizers.  All arithmetic is 64-bit where a
// product of caller sizes could leave the 32-bit range.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace dsa {
namespace plan {

// ---- top-k (topk.hip)
constexpr int kTopkBins = 4096;    // first / second digit histogram bins (12 bits)
constexpr int kTopkCoarse = 256;   // top 8 key bits: sign + 7 exponent bits
constexpr int kTopkCtrl = 4;       // per-row control words
constexpr int kTopkHeaderWords = kTopkBins + kTopkCoarse + kTopkCtrl;  // per-row words zeroed before each call
constexpr int kTopkChunk = 4096;       // slots per chunk of the chunked path (rows longer than this are chunked)
constexpr int kTopkChunkSmall = 2048;  // ... when kTopkChunk would give fewer than kTopkSmallGridWgs chunks
constexpr int kTopkSmallGridWgs = 512;
constexpr int kTopkChunkedMaxRows = 1024;  // from this many rows on, one workgroup per row fills the chip

// Few long rows: chunked over the whole chip; otherwise one workgroup per row.
inline bool topk_chunked(int32_t M, int32_t S_max) { return S_max > kTopkChunk && M < kTopkChunkedMaxRows; }

// Chunk size of the chunked path.
inline int topk_chunk(int32_t M, int32_t S_max)
{
    const long long n4 = (long long)M * (((long long)S_max + kTopkChunk - 1) / kTopkChunk);
    return n4 < kTopkSmallGridWgs ? kTopkChunkSmall : kTopkChunk;
}

// Per-chunk count pairs per row (sized for the smaller chunk).
inline size_t topk_count_words(int32_t S_max) { return ((size_t)S_max + kTopkChunkSmall - 1) / kTopkChunkSmall; }

// Workspace of the chunked path: row headers (zeroed before each call),
// per-chunk counts, candidate regions (one (key, slot) pair per slot).
inline size_t topk_workspace_bytes(int32_t M, int32_t S_max)
{
    if (!topk_chunked(M, S_max)) return 0;
    return (size_t)M * kTopkHeaderWords * 4 + (size_t)M * topk_count_words(S_max) * 8 + (size_t)M * S_max * 8;
}

// Leading 32-bit words of that workspace that must be zero when it starts.
inline size_t topk_header_words(int32_t M, int32_t S_max)
{
    return topk_chunked(M, S_max) ? (size_t)M * kTopkHeaderWords : 0;
}

// ---- sparse attention (sparse_attn_wide.hip, sparse_attn_decode.hip)
constexpr int kWideHeads = 128;         // heads per workgroup of the many-token kernel
constexpr int kWideMinWorkgroups = 256;  // it runs when its workgroups fill the chip
constexpr int kDecodeHeadsPerGroup = 64;  // heads per workgroup of the few-token kernel
constexpr int kDecodeBlock = 32;          // index-list entries per block
constexpr int kDecodeTargetGroups = 256;  // workgroups wanted to fill the chip
constexpr int kDecodeMaxSplits = 8;
constexpr int kDecodeMinSplitBlocks = 4;  // blocks per split at least

inline bool attn_wide(int32_t B, int32_t S, int32_t Hq)
{
    return (long long)B * S * (((long long)Hq + kWideHeads - 1) / kWideHeads) >= kWideMinWorkgroups;
}

// Parts the few-token kernel cuts each index list into: enough for about
// kDecodeTargetGroups workgroups, at most kDecodeMaxSplits, at least
// kDecodeMinSplitBlocks blocks each.
inline int attn_decode_splits(long long BS, int32_t Hq, int32_t K_top)
{
    const long long HG = ((long long)Hq + kDecodeHeadsPerGroup - 1) / kDecodeHeadsPerGroup;
    const long long groups = BS * HG;
    const long long nblk = ((long long)K_top + kDecodeBlock - 1) / kDecodeBlock;
    long long ns = (kDecodeTargetGroups + groups - 1) / groups;
    if (ns > kDecodeMaxSplits) ns = kDecodeMaxSplits;
    const long long by_blocks = nblk / kDecodeMinSplitBlocks > 1 ? nblk / kDecodeMinSplitBlocks : 1;
    if (ns > by_blocks) ns = by_blocks;
    return ns < 1 ? 1 : (int)ns;
}

// Partial results of the split lists: bf16 outputs (256-byte aligned), then
// one (max, sum) float pair per (token, split, head).
inline size_t attn_decode_partial_out_bytes(int32_t B, int32_t S, int32_t Hq, int32_t Dv, int ns)
{
    return ((size_t)B * S * ns * Hq * Dv * 2 + 255) & ~(size_t)255;
}

inline size_t attn_partial_bytes(int32_t B, int32_t S, int32_t Hq, int32_t Dv, int32_t K_top)
{
    if (attn_wide(B, S, Hq)) return 0;
    const int ns = attn_decode_splits((long long)B * S, Hq, K_top);
    if (ns <= 1) return 0;
    return attn_decode_partial_out_bytes(B, S, Hq, Dv, ns) + (size_t)B * S * ns * Hq * 8;
}

// ---- masked-dense attention (attn_masked_dense.hip): the dense slot list
// of every query token, then the attention's partials for a list of S_kv entries
inline size_t masked_dense_list_bytes(int32_t B, int32_t S, int32_t S_kv)
{
    return ((size_t)B * S * S_kv * 4 + 255) / 256 * 256;
}
inline size_t masked_dense_workspace_bytes(int32_t B, int32_t S, int32_t Hq, int32_t Dv, int32_t S_kv)
{
    return masked_dense_list_bytes(B, S, S_kv) + attn_partial_bytes(B, S, Hq, Dv, S_kv);
}

}  // namespace plan
}  // namespace dsa
