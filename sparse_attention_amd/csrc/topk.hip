// Top-k slot selection per score row for gfx950.
//
// Contract (AWS Neuron "DeepSeek-V3.2 Sparse Indexer Kernel API
// Reference", Returns and Notes): the index_topk highest-scoring attendable
// slots of each row, as an unordered set, padded with -1 when a row has
// fewer attendable slots.
//
// Both paths are radix selects on order-preserving 32-bit keys of the fp32
// scores (digits: key bits 31..20, 19..8, 7..0).  After each digit the
// bucket holding the k-th largest key is found by a suffix scan of the
// histogram; keys above it are selected, keys inside it stay candidates.
//
// The output is deterministic: every position is fixed by prefix sums over
// threads, waves and chunks in a fixed order (no atomic decides an output
// position), so repeated calls on the same scores return the same row,
// column for column, and ties at the final threshold are broken the same
// way every time.  The set contract would allow any order; a fixed one
// makes the attention that sums over the list bitwise reproducible.
//
//  * chunked path (few long rows, the decode case): rows are cut into
//    4096-slot chunks (2048 when that leaves fewer than 512 workgroups) so
//    the whole chip works on them.
//      topk_clear   zero the per-row histograms / counters in the workspace
//                   (the decode step has its scorer do this instead)
//      topk_hist    per chunk: LDS histogram of the first digit, flushed to
//                   the row's global histograms with atomics (non-zero
//                   bins): 4096 fine bins and 256 coarse bins (top 8 bits)
//                   so later stages find the threshold bin cheaply
//      topk_filter  per chunk: threshold bucket from the row histogram;
//                   the chunk's (key, slot) pairs above it, then those in
//                   it, go to the chunk's own region of the candidate
//                   buffer (positions from a workgroup scan), and their two
//                   counts to the row's count table; chunk 0 also records
//                   the row's threshold bin.  No global atomics;
//      topk_resolve one workgroup per row: prefix sums of the chunk counts
//                   place every chunk's slots above the threshold bin in
//                   the output in chunk order, then the two remaining
//                   digits run over the threshold bin's candidates.  Kernel
//                   boundaries make the other workgroups' writes visible; an
//                   in-kernel "last workgroup" hand-off would need a
//                   device-scope fence, which on these multi-XCD parts
//                   writes back the L2.
//  * row path (many short rows, e.g. prefill): one workgroup per row runs
//    all digits with LDS histograms; rows of up to 8192 slots are read once
//    into LDS, longer rows are re-read from memory per digit.
//
// The decode step uses the same kernels to emit its index list: with
// window > 0 a selected slot inside the window [n_valid - window, n_valid)
// is written as -1 and the window positions follow the top-k columns.
#include "device_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

// sizes shared with the host-side planning (launch_plan.h)
constexpr int kBins = plan::kTopkBins;  // first / second digit: 12 bits
constexpr int kChunk = plan::kTopkChunk;
constexpr int kChunkSmall = plan::kTopkChunkSmall;
constexpr int kChunkThreads = 256;
constexpr int kRowThreads = 1024;
constexpr int kCoarse = plan::kTopkCoarse;  // top 8 key bits: sign + 7 exponent bits
constexpr int kHeaderWords = plan::kTopkHeaderWords;  // per-row words zeroed before each call; control word
                                                      // kBins + kCoarse + 2 = threshold bin of the first digit
constexpr int kResolveCap = 8192;  // candidates resolved from LDS; more are re-read from HBM
constexpr int kRowLdsThreads = 512;
constexpr int kRowCap = 8192;      // row path: rows up to this many slots are held in LDS
constexpr int kMaxChunks = 4096;   // chunks per row the resolve's LDS prefix tables hold (rows up to 2^24 slots)

// ---------------------------------------------------------------- helpers

// Inclusive prefix sum over the 64 lanes of a wave on the DPP network: four
// row shifts within each 16-lane row, then rows 1 and 3 add lane 15 / 47 and
// rows 2 and 3 add lane 31 (no LDS round trips).
__device__ __forceinline__ int wave_scan_dpp(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return v;
}

// Number of lanes below this one whose bit is set in m.
__device__ __forceinline__ int lanes_below(uint64_t m)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Inclusive prefix sum over a workgroup of NT threads.
template <int NT>
__device__ __forceinline__ int block_inclusive_scan(int v, int* wave_tot)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    v = wave_scan_dpp(v);
    if (lane == 63) wave_tot[wave] = v;
    __syncthreads();
    int add = 0;
    for (int i = 0; i < wave; ++i) add += wave_tot[i];
    __syncthreads();
    return v + add;
}

// Digit d with above(d) < need <= above(d) + hist[d], where above(d) counts
// keys with a larger digit; result in *res_digit / *res_above (shared).
template <int NT>
__device__ void find_bucket(const int* hist, int nbins, int need, int* wave_tot, int* res_digit, int* res_above)
{
    const int per = nbins / NT > 0 ? nbins / NT : 1;
    const int top = nbins - 1 - (int)threadIdx.x * per;  // highest bin of this thread
    int local = 0;
    if (top >= 0)
        for (int i = 0; i < per; ++i) local += hist[top - i];
    const int incl = block_inclusive_scan<NT>(local, wave_tot);
    const int excl = incl - local;
    if (top >= 0 && excl < need && need <= incl) {
        int cum = excl;
        for (int i = 0; i < per; ++i) {
            const int h = hist[top - i];
            if (cum + h >= need) {
                *res_digit = top - i;
                *res_above = cum;
                break;
            }
            cum += h;
        }
    }
    __syncthreads();
}

__device__ __forceinline__ int emit(int s, int wstart) { return s >= wstart ? -1 : s; }

__device__ __forceinline__ float key_to_f32(uint32_t key)
{
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Deterministic output pass of a row path: wave w of NT / 64 owns the slot
// range [w * span, (w + 1) * span) (span a multiple of 256), a lane takes 4
// consecutive slots per step.  Each wave counts its slots above the final
// threshold (gt) and at it (eq); one barrier shares the counts; then each
// wave emits its range in slot order: gt slots from column (gt count of the
// lower waves), eq slots from n_gt + (eq count of the lower waves) while
// fewer than `remaining` are placed.  Ranks come from one ballot per slot
// phase (e = 0..3) and class, counted below each lane with mbcnt, so a
// step makes no cross-lane LDS round trip.  key4(s) gives the order keys of
// slots s .. s + 3 (s a multiple of 4; slots >= nv are never used); a
// position outside [0, k) is never written.
template <int NT, typename Key4>
__device__ __forceinline__ void emit_row(Key4 key4, int nv, uint32_t prefix, uint32_t pmask, int k,
                                         int remaining, int wstart, int (*wcnt)[NT / 64], int32_t* __restrict__ orow,
                                         float* __restrict__ osc)
{
    const int wave = threadIdx.x >> 6;
    const int span = ((nv + NT / 64 - 1) / (NT / 64) + 255) & ~255;
    const int lo = wave * span;
    const int hi = min(lo + span, nv);
    // per-slot-phase ballots: bit l of gt[e] / eq[e] is slot s0 + 4 l + e
    auto classify = [&](int s, u32x4 kk, uint64_t* gt, uint64_t* eq) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t km = kk[e] & pmask;
            const bool in = s + e < hi;
            gt[e] = __ballot(in && km > prefix);
            eq[e] = __ballot(in && km == prefix);
        }
    };
    int c_gt = 0, c_eq = 0;  // wave-uniform
    for (int s0 = lo; s0 < hi; s0 += 256) {
        const int s = s0 + 4 * (threadIdx.x & 63);
        const u32x4 kk = key4(s < hi ? s : lo);
        uint64_t gt[4], eq[4];
        classify(s, kk, gt, eq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            c_gt += __popcll(gt[e]);
            c_eq += __popcll(eq[e]);
        }
    }
    if ((threadIdx.x & 63) == 0) {
        wcnt[0][wave] = c_gt;
        wcnt[1][wave] = c_eq;
    }
    __syncthreads();
    int bgt = 0, beq = 0;
    for (int w = 0; w < wave; ++w) {
        bgt += wcnt[0][w];
        beq += wcnt[1][w];
    }
    const int n_gt = k - remaining;
    for (int s0 = lo; s0 < hi; s0 += 256) {
        const int s = s0 + 4 * (threadIdx.x & 63);
        const u32x4 kk = key4(s < hi ? s : lo);
        uint64_t gt[4], eq[4];
        classify(s, kk, gt, eq);
        int g = bgt, q = beq;  // this lane's first gt / eq rank
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            g += lanes_below(gt[e]);
            q += lanes_below(eq[e]);
        }
        const uint32_t lb = 1u << (threadIdx.x & 31);
        const int hl = (threadIdx.x >> 5) & 1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool is_gt = (uint32_t)(gt[e] >> (32 * hl)) & lb;
            const bool is_eq = (uint32_t)(eq[e] >> (32 * hl)) & lb;
            int pos = -1;
            if (is_gt) {
                pos = g++;
            } else if (is_eq) {
                if (q < remaining) pos = n_gt + q;
                ++q;
            }
            if (pos >= 0 && pos < k) {
                orow[pos] = emit(s + e, wstart);
                if (osc) osc[pos] = key_to_f32(kk[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bgt += __popcll(gt[e]);
            beq += __popcll(eq[e]);
        }
    }
}

// Deterministic compaction of one round of a workgroup of NT threads: this
// thread's rank among the round's `gt` threads and among its `eq` threads
// (lower waves first, then lower lanes), and the round's totals.  wcnt is a
// [2][2][NT / 64] LDS table used alternately by successive rounds (`parity`),
// so one barrier per round suffices.
template <int NT>
__device__ __forceinline__ void round_ranks(bool gt, bool eq, int (*wcnt)[2][NT / 64], int parity, int* rank_gt,
                                            int* rank_eq, int* tot_gt, int* tot_eq)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;  // lanes below this one
    const uint64_t bg = __ballot(gt);
    const uint64_t be = __ballot(eq);
    if (lane == 0) {
        wcnt[parity][0][wave] = __popcll(bg);
        wcnt[parity][1][wave] = __popcll(be);
    }
    __syncthreads();
    int bgt = 0, beq = 0, tg = 0, te = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const int a = wcnt[parity][0][w];
        const int b = wcnt[parity][1][w];
        bgt += w < wave ? a : 0;
        beq += w < wave ? b : 0;
        tg += a;
        te += b;
    }
    *rank_gt = bgt + __popcll(bg & lt);
    *rank_eq = beq + __popcll(be & lt);
    *tot_gt = tg;
    *tot_eq = te;
}

// ---------------------------------------------------------------- row path

__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(
    const float* __restrict__ scores, int32_t S_max, const int32_t* __restrict__ positions, int32_t valid_len,
    int32_t k, int32_t window, int32_t* __restrict__ out_idx, float* __restrict__ out_scores)
{
    __shared__ int hist[kBins];
    __shared__ int wave_tot[kRowThreads / 64];
    __shared__ int wcnt[2][kRowThreads / 64];
    __shared__ int sh_digit, sh_above;

    const int r = blockIdx.x;
    const int nv = n_valid_of(positions, valid_len, r, S_max);
    const int width = k + window;
    const int wstart = nv - window;
    const float* __restrict__ row = scores + (size_t)r * S_max;
    int32_t* __restrict__ orow = out_idx + (size_t)r * width;
    float* __restrict__ osc = out_scores ? out_scores + (size_t)r * k : nullptr;
    const int t = threadIdx.x;

    for (int i = t; i < window; i += kRowThreads) {
        const int p = wstart + i;
        orow[k + i] = p < 0 ? -1 : p;
    }
    if (nv <= k) {
        for (int j = t; j < k; j += kRowThreads) {
            const int s = j < nv ? j : -1;
            orow[j] = s < 0 ? -1 : emit(s, wstart);
            if (osc) osc[j] = s >= 0 ? row[s] : -INFINITY;
        }
        return;
    }

    uint32_t prefix = 0, pmask = 0;
    int remaining = k;
    const int shifts[3] = {20, 8, 0};
    const int bits[3] = {12, 12, 8};
    for (int pass = 0; pass < 3; ++pass) {
        const int nb = 1 << bits[pass];
        const int sh = shifts[pass];
        for (int i = t; i < nb; i += kRowThreads) hist[i] = 0;
        __syncthreads();
        for (int s = t; s < nv; s += kRowThreads) {
            const uint32_t key = f32_order_key(row[s]);
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & (nb - 1)], 1);
        }
        __syncthreads();
        find_bucket<kRowThreads>(hist, nb, remaining, wave_tot, &sh_digit, &sh_above);
        const int d = sh_digit;
        remaining -= sh_above;
        prefix |= (uint32_t)d << sh;
        pmask |= (uint32_t)(nb - 1) << sh;
        const bool exact = hist[d] == remaining;
        __syncthreads();
        if (exact) break;
    }

    // (rows of this path may have any length: the four slots are read one by one, those past n_valid not at all)
    emit_row<kRowThreads>(
        [&](int s) {
            u32x4 kk;
#pragma unroll
            for (int e = 0; e < 4; ++e) kk[e] = s + e < nv ? f32_order_key(row[s + e]) : 0u;
            return kk;
        },
        nv, prefix, pmask, k, remaining, wstart, wcnt, orow, osc);
}

// Row path for rows of at most kRowCap slots (16-byte aligned): the row is
// read once with 16-byte loads, all of a thread's loads in flight before the
// first wait, into LDS as order keys, building the first digit's histogram
// on the way; later digits (16-byte LDS reads) and the output pass run on
// LDS.  Outputs are placed in slot order by emit_row (one barrier per row).
__global__ __launch_bounds__(kRowLdsThreads) void topk_row_lds_kernel(
    const float* __restrict__ scores, int32_t S_max, const int32_t* __restrict__ positions, int32_t valid_len,
    int32_t k, int32_t window, int32_t* __restrict__ out_idx, float* __restrict__ out_scores)
{
    constexpr int NT = kRowLdsThreads;
    __shared__ __attribute__((aligned(16))) uint32_t keys[kRowCap];
    __shared__ int hist[kBins];
    __shared__ int wave_tot[NT / 64];
    __shared__ int wcnt[2][NT / 64];
    __shared__ int sh_digit, sh_above;

    const int r = (int)(gridDim.x - 1 - blockIdx.x);  // long rows first
    const int nv = n_valid_of(positions, valid_len, r, S_max);
    const int width = k + window;
    const int wstart = nv - window;
    const float* __restrict__ row = scores + (size_t)r * S_max;
    int32_t* __restrict__ orow = out_idx + (size_t)r * width;
    float* __restrict__ osc = out_scores ? out_scores + (size_t)r * k : nullptr;
    const int t = threadIdx.x;

    for (int i = t; i < window; i += NT) {
        const int p = wstart + i;
        orow[k + i] = p < 0 ? -1 : p;
    }
    if (nv <= k) {
        for (int j = t; j < k; j += NT) {
            const int s = j < nv ? j : -1;
            orow[j] = s < 0 ? -1 : emit(s, wstart);
            if (osc) osc[j] = s >= 0 ? row[s] : -INFINITY;
        }
        return;
    }

    for (int i = t; i < kBins; i += NT) hist[i] = 0;
    __syncthreads();
    const int nv4 = (nv + 3) & ~3;  // <= S_max (a multiple of 4)
    {
        // every load of the row in flight at once (addresses clamped into the row), then the keys
        constexpr int kPer = kRowCap / (4 * NT);
        u32x4 v[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int s = 4 * t + i * 4 * NT;
            v[i] = *reinterpret_cast<const u32x4*>(row + (s < nv4 ? s : 0));
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int s = 4 * t + i * 4 * NT;
            if (s < nv4) {
                u32x4 kk;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t key = f32_order_key(__uint_as_float(v[i][e]));
                    kk[e] = key;
                    if (s + e < nv) atomicAdd(&hist[key >> 20], 1);
                }
                *reinterpret_cast<u32x4*>(keys + s) = kk;
            }
        }
    }
    __syncthreads();

    uint32_t prefix = 0, pmask = 0;
    int remaining = k;
    const int shifts[3] = {20, 8, 0};
    const int bits[3] = {12, 12, 8};
    for (int pass = 0; pass < 3; ++pass) {
        const int nb = 1 << bits[pass];
        const int sh = shifts[pass];
        if (pass > 0) {
            for (int i = t; i < nb; i += NT) hist[i] = 0;
            __syncthreads();
            for (int s = 4 * t; s < nv4; s += 4 * NT) {
                const u32x4 kk = *reinterpret_cast<const u32x4*>(keys + s);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (s + e < nv && (kk[e] & pmask) == prefix) atomicAdd(&hist[(kk[e] >> sh) & (nb - 1)], 1);
            }
            __syncthreads();
        }
        find_bucket<NT>(hist, nb, remaining, wave_tot, &sh_digit, &sh_above);
        const int d = sh_digit;
        remaining -= sh_above;
        prefix |= (uint32_t)d << sh;
        pmask |= (uint32_t)(nb - 1) << sh;
        const bool exact = hist[d] == remaining;
        __syncthreads();
        if (exact) break;
    }

    emit_row<NT>([&](int s) { return *reinterpret_cast<const u32x4*>(keys + s); }, nv, prefix, pmask, k, remaining,
                 wstart, wcnt, orow, osc);
}

// ---------------------------------------------------------------- chunked path

// Zero n_quads 16-byte units (the header is a whole number of them per row
// and the workspace is 16-byte aligned).
__global__ __launch_bounds__(256) void topk_clear_kernel(u32x4* __restrict__ ws, int32_t n_quads)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n_quads) ws[i] = u32x4{0u, 0u, 0u, 0u};
}
static_assert(kHeaderWords % 4 == 0, "the header clear writes 16-byte units");

template <int CHUNK>
__global__ __launch_bounds__(kChunkThreads) void topk_hist_kernel(
    const float* __restrict__ scores, int32_t S_max, const int32_t* __restrict__ positions, int32_t valid_len,
    int32_t k, uint32_t* __restrict__ ghist)
{
    static_assert(kChunkThreads == kCoarse, "one thread per coarse bin");
    __shared__ int hist[kBins];
    const int r = blockIdx.y;
    const int s0 = blockIdx.x * CHUNK;
    const float* __restrict__ row = scores + (size_t)r * S_max;
    // The chunk's scores are loaded before n_valid is known (every slot
    // below S_max is readable), so the position lookup overlaps them.
    constexpr int kPer = CHUNK / kChunkThreads;  // slots per thread: loads first, then LDS atomics
    const int sl = min(s0 + CHUNK, S_max);
    float v[kPer];
    // 16-byte loads when the row is 16-byte aligned (slots s0 + 4 (i * NT + t) + e), else 4-byte ones
    const bool wide = ((reinterpret_cast<uintptr_t>(row) | (uintptr_t)S_max * 4) & 15) == 0;
    auto slot_of = [&](int i) {
        return wide ? s0 + 4 * ((i >> 2) * kChunkThreads + (int)threadIdx.x) + (i & 3) : s0 + i * kChunkThreads + (int)threadIdx.x;
    };
    if (wide) {
#pragma unroll
        for (int i = 0; i < kPer; i += 4) {
            const int s = slot_of(i);
            const float4 x = s < sl ? *reinterpret_cast<const float4*>(row + s) : float4{0.f, 0.f, 0.f, 0.f};
            v[i] = x.x; v[i + 1] = x.y; v[i + 2] = x.z; v[i + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int s = slot_of(i);
            v[i] = s < sl ? row[s] : 0.f;
        }
    }
    const int nv = n_valid_of(positions, valid_len, r, S_max);
    if (nv <= k || s0 >= nv) return;  // uniform
    const int s1 = min(s0 + CHUNK, nv);
    for (int i = threadIdx.x; i < kBins; i += kChunkThreads) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        if (slot_of(i) < s1) atomicAdd(&hist[f32_order_key(v[i]) >> 20], 1);
    __syncthreads();
    uint32_t* __restrict__ gh = ghist + (size_t)r * kHeaderWords;
    for (int i = threadIdx.x; i < kBins; i += kChunkThreads) {
        const int h = hist[i];
        if (h) atomicAdd(&gh[i], (uint32_t)h);
    }
    // coarse bin c = sum of fine bins 16c .. 16c + 15 (one thread per coarse bin)
    {
        const int c = threadIdx.x;  // kChunkThreads == kCoarse
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += hist[16 * c + ((i + c) & 15)];
        if (sum) atomicAdd(&gh[kBins + c], (uint32_t)sum);
    }
}

// Threshold bucket of the first digit from the row's two-level histogram:
// the coarse bin holding the k-th largest key, then the fine bin inside it.
// `coarse` is this thread's coarse bin, gh[kBins + threadIdx.x], loaded by
// the caller ahead of time.
__device__ void row_threshold(const uint32_t* __restrict__ gh, uint32_t coarse, int k, int* scratch, int* wave_tot,
                              int* res_digit, int* res_above)
{
    // coarse: 256 bins, one per thread
    scratch[threadIdx.x] = (int)coarse;
    __syncthreads();
    find_bucket<kChunkThreads>(scratch, kCoarse, k, wave_tot, res_digit, res_above);
    const int c1 = *res_digit;
    const int above_c = *res_above;
    __syncthreads();
    if (threadIdx.x < 16) scratch[threadIdx.x] = (int)gh[16 * c1 + threadIdx.x];
    __syncthreads();
    if (threadIdx.x == 0) {
        int cum = above_c;
        for (int i = 15; i >= 0; --i) {
            const int h = scratch[i];
            if (cum + h >= k) {
                *res_digit = 16 * c1 + i;
                *res_above = cum;
                break;
            }
            cum += h;
        }
    }
    __syncthreads();
}

template <int CHUNK>
__global__ __launch_bounds__(kChunkThreads) void topk_filter_kernel(
    const float* __restrict__ scores, int32_t S_max, const int32_t* __restrict__ positions, int32_t valid_len,
    int32_t k, int32_t window, uint32_t* __restrict__ ghist, int2* __restrict__ counts, int32_t n_counts,
    int2* __restrict__ cand, int32_t* __restrict__ out_idx, float* __restrict__ out_scores)
{
    __shared__ int scratch[kCoarse];
    __shared__ int wave_tot[kChunkThreads / 64];
    __shared__ int sh_digit, sh_above;

    const int r = blockIdx.y;
    const int nchunks = gridDim.x;
    const int s0 = blockIdx.x * CHUNK;
    const float* __restrict__ row = scores + (size_t)r * S_max;
    const int t = threadIdx.x;
    // Loads that do not depend on n_valid go first (every slot below S_max
    // is readable): this chunk's scores and this thread's coarse bin, so that
    // the position lookup, the scores and the threshold lookup share one
    // memory latency.
    constexpr int kPer = CHUNK / kChunkThreads;  // slots per thread
    const int sl = min(s0 + CHUNK, S_max);
    float v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int s = s0 + i * kChunkThreads + t;
        v[i] = s < sl ? row[s] : 0.f;
    }
    uint32_t* __restrict__ gh = ghist + (size_t)r * kHeaderWords;
    const uint32_t coarse = gh[kBins + t];  // kChunkThreads == kCoarse
    const int nv = n_valid_of(positions, valid_len, r, S_max);
    const int width = k + window;
    const int wstart = nv - window;
    int32_t* __restrict__ orow = out_idx + (size_t)r * width;
    float* __restrict__ osc = out_scores ? out_scores + (size_t)r * k : nullptr;

    if (blockIdx.x == 0)
        for (int i = t; i < window; i += kChunkThreads) {
            const int p = wstart + i;
            orow[k + i] = p < 0 ? -1 : p;
        }
    if (nv <= k) {
        // every attendable slot is selected, in slot order; -1 pads the rest
        for (int j = s0 + t; j < min(s0 + CHUNK, k); j += kChunkThreads) {
            const int s = j < nv ? j : -1;
            orow[j] = s < 0 ? -1 : emit(s, wstart);
            if (osc) osc[j] = s >= 0 ? row[s] : -INFINITY;
        }
        if (blockIdx.x == nchunks - 1)  // k may exceed the chunked range
            for (int j = nchunks * CHUNK + t; j < k; j += kChunkThreads) {
                orow[j] = -1;
                if (osc) osc[j] = -INFINITY;
            }
        return;
    }
    if (s0 >= nv) return;  // uniform: the resolve reads only chunks below n_valid (chunk 0 always runs)

    const int s1 = min(s0 + CHUNK, nv);
    uint32_t keys[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int s = s0 + i * kChunkThreads + t;
        keys[i] = (s < s1) ? f32_order_key(v[i]) : 0u;
    }
    row_threshold(gh, coarse, k, scratch, wave_tot, &sh_digit, &sh_above);
    const uint32_t d1 = (uint32_t)sh_digit;
    if (blockIdx.x == 0 && t == 0) gh[kBins + kCoarse + 2] = d1;  // for the resolve (visible after this kernel)

    int my_gt = 0, my_eq = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const bool in = s0 + i * kChunkThreads + t < s1;
        const uint32_t dg = keys[i] >> 20;
        my_gt += (in && dg > d1) ? 1 : 0;
        my_eq += (in && dg == d1) ? 1 : 0;
    }
    // both counts in one scan: at most CHUNK <= 2^15 each, so the halves never carry into each other
    const int packed = my_gt | (my_eq << 16);
    const int incl = block_inclusive_scan<kChunkThreads>(packed, wave_tot);
    int tot = 0;
#pragma unroll
    for (int i = 0; i < kChunkThreads / 64; ++i) tot += wave_tot[i];
    const int excl = incl - packed;
    const int tot_gt = tot & 0xFFFF;
    int off_gt = excl & 0xFFFF;
    int off_eq = tot_gt + (excl >> 16);
    // the chunk's region: slots above the threshold bin first, then the bin's candidates
    int2* __restrict__ region = cand + (size_t)r * S_max + s0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int s = s0 + i * kChunkThreads + t;
        if (s >= s1) continue;
        const uint32_t dg = keys[i] >> 20;
        if (dg > d1) region[off_gt++] = make_int2((int)keys[i], s);
        else if (dg == d1) region[off_eq++] = make_int2((int)keys[i], s);
    }
    if (t == 0) counts[(size_t)r * n_counts + blockIdx.x] = make_int2(tot_gt, tot >> 16);
}

// Per row: the chunks' slots above the threshold bin go to the output in
// chunk order; the threshold bin's candidates (gathered in chunk order, in
// LDS when they fit) are resolved with the two remaining digits and placed
// by per-round ranks.
template <int CHUNK>
__global__ __launch_bounds__(kChunkThreads) void topk_resolve_kernel(
    const float* __restrict__ scores, int32_t S_max, const int32_t* __restrict__ positions, int32_t valid_len,
    int32_t k, int32_t window, const uint32_t* __restrict__ ghist, const int2* __restrict__ counts,
    int32_t n_counts, const int2* __restrict__ cand, int32_t* __restrict__ out_idx, float* __restrict__ out_scores)
{
    constexpr int NT = kChunkThreads;
    __shared__ int hist[kBins];
    __shared__ int2 lcand[kResolveCap];
    __shared__ int pre_gt[kMaxChunks + 1];  // exclusive prefix sums of the chunks' counts
    __shared__ int pre_eq[kMaxChunks + 1];
    __shared__ int wave_tot[NT / 64];
    __shared__ long long wave_tot64[NT / 64];
    __shared__ int wcnt[2][2][NT / 64];
    __shared__ int sh_digit, sh_above;

    const int r = blockIdx.x;
    const int t = threadIdx.x;
    const int2* __restrict__ crow = counts + (size_t)r * n_counts;
    // the threshold bin, the first NT chunk counts and the position, read together
    const uint32_t d1 = ghist[(size_t)r * kHeaderWords + kBins + kCoarse + 2];
    const int2 n_first = t < n_counts ? crow[t] : make_int2(0, 0);
    const int nv = n_valid_of(positions, valid_len, r, S_max);
    if (nv <= k) return;  // uniform
    const int width = k + window;
    const int wstart = nv - window;
    int32_t* __restrict__ orow = out_idx + (size_t)r * width;
    float* __restrict__ osc = out_scores ? out_scores + (size_t)r * k : nullptr;
    const int nch = (nv + CHUNK - 1) / CHUNK;  // chunks the filter filled (<= kMaxChunks)
    const int2* __restrict__ rbase = cand + (size_t)r * S_max;

    // prefix sums of the chunk counts (both counts in one 64-bit scan), 256 chunks per round
    long long carry = 0;  // gt total | eq total << 32
    for (int c0 = 0; c0 < nch; c0 += NT) {
        const int c = c0 + t;
        const int2 n = c >= nch ? make_int2(0, 0) : (c0 == 0 ? n_first : crow[c]);
        // each count of a row is below 2^24: two 32-bit wave scans, packed after
        const long long x = (long long)(uint32_t)wave_scan_dpp(n.x) | ((long long)wave_scan_dpp(n.y) << 32);
        if ((t & 63) == 63) wave_tot64[t >> 6] = x;
        __syncthreads();
        long long add = carry, tot = carry;
#pragma unroll
        for (int i = 0; i < NT / 64; ++i) {
            add += i < (t >> 6) ? wave_tot64[i] : 0;
            tot += wave_tot64[i];
        }
        if (c < nch) {
            pre_gt[c + 1] = (int)(add + x);
            pre_eq[c + 1] = (int)((add + x) >> 32);
        }
        carry = tot;
        __syncthreads();
    }
    if (t == 0) {
        pre_gt[0] = 0;
        pre_eq[0] = 0;
    }
    __syncthreads();
    const int total_gt = (int)carry;     // slots above the threshold bin
    const int n_cand = (int)(carry >> 32);  // slots in it
    // chunk holding entry j of a prefix table: the largest c with pre[c] <= j
    auto chunk_of = [&](const int* pre, int j) -> int {
        int lo = 0, hi = nch;  // pre[lo] <= j < pre[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (pre[mid] <= j) lo = mid;
            else hi = mid;
        }
        return lo;
    };
    // i-th candidate of the threshold bin, in chunk order
    auto cand_global = [&](int i) -> int2 {
        const int c = chunk_of(pre_eq, i);
        return rbase[c * CHUNK + (pre_gt[c + 1] - pre_gt[c]) + (i - pre_eq[c])];
    };

    // Source index (in the row's candidate regions) of every entry, written
    // by the wave that owns the chunk: above-threshold entries into hist
    // (free until the digit passes; total_gt < k <= kBins), bin candidates
    // into lcand[].x when they fit in LDS.
    const bool in_lds = n_cand <= kResolveCap;
    {
        const int lane = t & 63;
        for (int c = t >> 6; c < nch; c += NT / 64) {
            const int g0 = pre_gt[c], ng = pre_gt[c + 1] - g0;
            for (int i = lane; i < ng; i += 64) hist[g0 + i] = c * CHUNK + i;
            if (in_lds) {
                const int e0 = pre_eq[c], ne = pre_eq[c + 1] - e0;
                for (int i = lane; i < ne; i += 64) lcand[e0 + i].x = c * CHUNK + ng + i;
            }
        }
    }
    __syncthreads();
    // The slots above the threshold bin go to output columns [0, total_gt) in
    // chunk order; the first candidates come into LDS.  All loads are issued
    // before the first store.
    constexpr int kMaxPer = DSA_MAX_TOPK / NT;
    int2 ea[kMaxPer], ec[kMaxPer];
    // Every lane loads (entry 0 of the row's regions where it has nothing to
    // fetch), so no branch surrounds a load and all of them are in flight
    // together; with per-lane branches each load drained the previous ones.
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u) {
        const int j = t + u * NT;
        const bool oka = j < total_gt, okc = in_lds && j < n_cand;
        const int ia = hist[j];                              // j < kMaxPer * NT <= kBins
        const int ic = lcand[j < kResolveCap ? j : 0].x;
        const int2 va = rbase[oka ? ia : 0];
        const int2 vc = rbase[okc ? ic : 0];
        ea[u] = oka ? va : make_int2(0, -1);
        ec[u] = okc ? vc : make_int2(0, 0);
    }
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u) {
        const int j = t + u * NT;
        if (j < total_gt) {
            orow[j] = emit(ea[u].y, wstart);
            if (osc) osc[j] = key_to_f32((uint32_t)ea[u].x);
        }
        if (in_lds && j < n_cand) lcand[j] = ec[u];
    }
    if (in_lds)  // candidates beyond the first kMaxPer * NT (each thread rewrites only its own entries)
        for (int i = t + kMaxPer * NT; i < n_cand; i += NT) lcand[i] = rbase[lcand[i].x];
    __syncthreads();
    auto cand_at = [&](int i) -> int2 { return in_lds ? lcand[i] : cand_global(i); };

    int remaining = k - total_gt;
    uint32_t prefix = d1 << 20, pmask = 0xFFF00000u;
    if (remaining < n_cand) {
        const int shifts[2] = {8, 0};
        const int bits[2] = {12, 8};
        for (int pass = 0; pass < 2; ++pass) {
            const int nb = 1 << bits[pass];
            const int sh = shifts[pass];
            for (int i = t; i < nb; i += NT) hist[i] = 0;
            __syncthreads();
            for (int i = t; i < n_cand; i += NT) {
                const uint32_t key = (uint32_t)cand_at(i).x;
                if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & (nb - 1)], 1);
            }
            __syncthreads();
            find_bucket<NT>(hist, nb, remaining, wave_tot, &sh_digit, &sh_above);
            const int d = sh_digit;
            remaining -= sh_above;
            prefix |= (uint32_t)d << sh;
            pmask |= (uint32_t)(nb - 1) << sh;
            const bool exact = hist[d] == remaining;
            __syncthreads();
            if (exact) break;
        }
    }
    const int n_gt = k - remaining;  // slots already placed or strictly above the final threshold
    int cg = 0, ce = 0, parity = 0;
    for (int i0 = 0; i0 < n_cand; i0 += NT) {  // uniform trip count
        const int i = i0 + t;
        int2 ck = make_int2(0, 0);
        if (i < n_cand) ck = cand_at(i);
        const uint32_t km = (uint32_t)ck.x & pmask;
        const bool gt = i < n_cand && km > prefix;
        const bool eq = i < n_cand && km == prefix;
        int rg, re, tg, te;
        round_ranks<NT>(gt, eq, wcnt, parity, &rg, &re, &tg, &te);
        int pos = -1;
        if (gt) {
            pos = total_gt + cg + rg;
        } else if (eq) {
            const int tk = ce + re;
            if (tk < remaining) pos = n_gt + tk;
        }
        if (pos >= 0) {
            orow[pos] = emit(ck.y, wstart);
            if (osc) osc[pos] = key_to_f32((uint32_t)ck.x);
        }
        cg += tg;
        ce += te;
        parity ^= 1;
    }
}


}  // namespace

hipError_t launch_topk(const float* scores, int32_t M, int32_t S_max, const int32_t* positions,
                       int32_t valid_len, int32_t k, int32_t window, int32_t* out_idx, float* out_scores,
                       void* workspace, bool header_zeroed, hipStream_t stream)
{
    if (!plan::topk_chunked(M, S_max)) {
        if (S_max <= kRowCap && (S_max & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0)
            topk_row_lds_kernel<<<M, kRowLdsThreads, 0, stream>>>(scores, S_max, positions, valid_len, k, window,
                                                                  out_idx, out_scores);
        else
            topk_row_kernel<<<M, kRowThreads, 0, stream>>>(scores, S_max, positions, valid_len, k, window, out_idx,
                                                           out_scores);
        return hipGetLastError();
    }
    uint32_t* ghist = static_cast<uint32_t*>(workspace);
    const int n_counts = (int)plan::topk_count_words(S_max);
    int2* counts = reinterpret_cast<int2*>(ghist + (size_t)M * kHeaderWords);
    int2* cand = counts + (size_t)M * n_counts;
    const int n_quads = M * (kHeaderWords / 4);
    if (!header_zeroed)
        topk_clear_kernel<<<(n_quads + 255) / 256, 256, 0, stream>>>(reinterpret_cast<u32x4*>(ghist), n_quads);
    // chunk size: 4096 slots, or 2048 when that would leave the chip short of workgroups
    if (plan::topk_chunk(M, S_max) == kChunkSmall) {
        const dim3 grid((S_max + kChunkSmall - 1) / kChunkSmall, M);
        topk_hist_kernel<kChunkSmall><<<grid, kChunkThreads, 0, stream>>>(scores, S_max, positions, valid_len, k, ghist);
        topk_filter_kernel<kChunkSmall><<<grid, kChunkThreads, 0, stream>>>(
            scores, S_max, positions, valid_len, k, window, ghist, counts, n_counts, cand, out_idx, out_scores);
        topk_resolve_kernel<kChunkSmall><<<M, kChunkThreads, 0, stream>>>(
            scores, S_max, positions, valid_len, k, window, ghist, counts, n_counts, cand, out_idx, out_scores);
    } else {
        const dim3 grid((S_max + kChunk - 1) / kChunk, M);
        topk_hist_kernel<kChunk><<<grid, kChunkThreads, 0, stream>>>(scores, S_max, positions, valid_len, k, ghist);
        topk_filter_kernel<kChunk><<<grid, kChunkThreads, 0, stream>>>(
            scores, S_max, positions, valid_len, k, window, ghist, counts, n_counts, cand, out_idx, out_scores);
        topk_resolve_kernel<kChunk><<<M, kChunkThreads, 0, stream>>>(
            scores, S_max, positions, valid_len, k, window, ghist, counts, n_counts, cand, out_idx, out_scores);
    }
    return hipGetLastError();
}

}  // namespace dsa
