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
// Ties at the final threshold are taken in arrival order, which the set
// contract allows.
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
//                   slots above it are written out directly (one global
//                   atomic per workgroup reserves the output range), slots
//                   in it are appended to the row's (key, slot) list;
//                   chunk 0 also records the row's threshold bin and the
//                   count above it for the resolve;
//      topk_resolve one workgroup per row runs the two remaining digits over
//                   the candidates.  Kernel boundaries make the other
//                   workgroups' writes visible; an in-kernel "last
//                   workgroup" hand-off would need a device-scope fence,
//                   which on these multi-XCD parts writes back the L2.
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

constexpr int kBins = 4096;  // first / second digit: 12 bits
constexpr int kChunk = 4096;  // slots per workgroup in the chunked path (rows longer than this are chunked)
constexpr int kChunkSmall = 2048;  // ... when 4096-slot chunks would give fewer than kSmallGridWgs workgroups
constexpr int kSmallGridWgs = 512;
constexpr int kChunkThreads = 256;
constexpr int kRowThreads = 1024;
constexpr int kCoarse = 256;  // top 8 key bits: sign + 7 exponent bits
constexpr int kCtrl = 4;      // per-row words: above-threshold count, candidate count, threshold bin, count above it
constexpr int kHeaderWords = kBins + kCoarse + kCtrl;  // per-row words zeroed before each call
constexpr int kResolveCap = 8192;  // candidates resolved from LDS; more are re-read from HBM
constexpr int kRowLdsThreads = 512;
constexpr int kRowCap = 8192;      // row path: rows up to this many slots are held in LDS

// ---------------------------------------------------------------- helpers

// Inclusive prefix sum over a workgroup of NT threads.
template <int NT>
__device__ __forceinline__ int block_inclusive_scan(int v, int* wave_tot)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(v, off, 64);
        if (lane >= off) v += t;
    }
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

// ---------------------------------------------------------------- row path

__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(
    const float* __restrict__ scores, int32_t S_max, const int32_t* __restrict__ positions, int32_t valid_len,
    int32_t k, int32_t window, int32_t* __restrict__ out_idx, float* __restrict__ out_scores)
{
    __shared__ int hist[kBins];
    __shared__ int wave_tot[kRowThreads / 64];
    __shared__ int sh_digit, sh_above, cnt_gt, cnt_eq;

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

    if (t == 0) {
        cnt_gt = 0;
        cnt_eq = 0;
    }
    __syncthreads();
    const int n_gt = k - remaining;
    for (int s = t; s < nv; s += kRowThreads) {
        const float v = row[s];
        const uint32_t km = f32_order_key(v) & pmask;
        int pos = -1;
        if (km > prefix) {
            pos = atomicAdd(&cnt_gt, 1);
        } else if (km == prefix) {
            const int tk = atomicAdd(&cnt_eq, 1);
            if (tk < remaining) pos = n_gt + tk;
        }
        if (pos >= 0) {
            orow[pos] = emit(s, wstart);
            if (osc) osc[pos] = v;
        }
    }
}

// Row path for rows of at most kRowCap slots (16-byte aligned): the row is
// read once with 16-byte loads into LDS as order keys, building the first
// digit's histogram on the way; later digits and the output pass run on LDS.
// Outputs are compacted per wave (ballot + one LDS atomic per wave).
__global__ __launch_bounds__(kRowLdsThreads) void topk_row_lds_kernel(
    const float* __restrict__ scores, int32_t S_max, const int32_t* __restrict__ positions, int32_t valid_len,
    int32_t k, int32_t window, int32_t* __restrict__ out_idx, float* __restrict__ out_scores)
{
    constexpr int NT = kRowLdsThreads;
    __shared__ __attribute__((aligned(16))) uint32_t keys[kRowCap];
    __shared__ int hist[kBins];
    __shared__ int wave_tot[NT / 64];
    __shared__ int sh_digit, sh_above, cnt_gt, cnt_eq;

    const int r = (int)(gridDim.x - 1 - blockIdx.x);  // long rows first
    const int nv = n_valid_of(positions, valid_len, r, S_max);
    const int width = k + window;
    const int wstart = nv - window;
    const float* __restrict__ row = scores + (size_t)r * S_max;
    int32_t* __restrict__ orow = out_idx + (size_t)r * width;
    float* __restrict__ osc = out_scores ? out_scores + (size_t)r * k : nullptr;
    const int t = threadIdx.x;
    const int lane = t & 63;

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
    for (int s = 4 * t; s < nv4; s += 4 * NT) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(row + s);
        u32x4 kk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t key = f32_order_key(__uint_as_float(v[e]));
            kk[e] = key;
            if (s + e < nv) atomicAdd(&hist[key >> 20], 1);
        }
        *reinterpret_cast<u32x4*>(keys + s) = kk;
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
            for (int s = t; s < nv; s += NT) {
                const uint32_t key = keys[s];
                if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & (nb - 1)], 1);
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

    if (t == 0) {
        cnt_gt = 0;
        cnt_eq = 0;
    }
    __syncthreads();
    const int n_gt = k - remaining;
    const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;  // lanes below this one
    for (int s0 = 0; s0 < nv; s0 += NT) {
        const int s = s0 + t;
        uint32_t key = 0;
        bool gt = false, eq = false;
        if (s < nv) {
            key = keys[s];
            gt = (key & pmask) > prefix;
            eq = (key & pmask) == prefix;
        }
        const uint64_t bg = __ballot(gt);
        const uint64_t be = __ballot(eq);
        int bgt = 0, beq = 0;
        if (lane == 0) {
            if (bg) bgt = atomicAdd(&cnt_gt, __popcll(bg));
            if (be) beq = atomicAdd(&cnt_eq, __popcll(be));
        }
        bgt = __shfl(bgt, 0, 64);
        beq = __shfl(beq, 0, 64);
        int pos = -1;
        if (gt) {
            pos = bgt + __popcll(bg & lt);
        } else if (eq) {
            const int tk = beq + __popcll(be & lt);
            if (tk < remaining) pos = n_gt + tk;
        }
        if (pos >= 0) {
            orow[pos] = emit(s, wstart);
            if (osc) osc[pos] = __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
        }
    }
}

// ---------------------------------------------------------------- chunked path

__global__ __launch_bounds__(256) void topk_clear_kernel(uint32_t* __restrict__ ws, int32_t n_words)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n_words) ws[i] = 0u;
}

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
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int s = s0 + i * kChunkThreads + (int)threadIdx.x;
        v[i] = s < sl ? row[s] : 0.f;
    }
    const int nv = n_valid_of(positions, valid_len, r, S_max);
    if (nv <= k || s0 >= nv) return;  // uniform
    const int s1 = min(s0 + CHUNK, nv);
    for (int i = threadIdx.x; i < kBins; i += kChunkThreads) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        if (s0 + i * kChunkThreads + (int)threadIdx.x < s1) atomicAdd(&hist[f32_order_key(v[i]) >> 20], 1);
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
    int32_t k, int32_t window, uint32_t* __restrict__ ghist, int2* __restrict__ cand,
    int32_t* __restrict__ out_idx, float* __restrict__ out_scores)
{
    __shared__ int scratch[kCoarse];
    __shared__ int wave_tot[kChunkThreads / 64];
    __shared__ int sh_digit, sh_above, cnt_gt, cnt_eq, base_gt, base_eq;

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

    const int s1 = min(s0 + CHUNK, nv);
    uint32_t keys[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int s = s0 + i * kChunkThreads + t;
        keys[i] = (s < s1) ? f32_order_key(v[i]) : 0u;
    }
    if (t == 0) {
        cnt_gt = 0;
        cnt_eq = 0;
    }
    row_threshold(gh, coarse, k, scratch, wave_tot, &sh_digit, &sh_above);
    const uint32_t d1 = (uint32_t)sh_digit;
    uint32_t* __restrict__ ctrl = gh + kBins + kCoarse;
    if (blockIdx.x == 0 && t == 0) {  // for the resolve (visible after this kernel)
        ctrl[2] = d1;
        ctrl[3] = (uint32_t)sh_above;
    }

    int my_gt = 0, my_eq = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const bool in = s0 + i * kChunkThreads + t < s1;
        const uint32_t dg = keys[i] >> 20;
        my_gt += (in && dg > d1) ? 1 : 0;
        my_eq += (in && dg == d1) ? 1 : 0;
    }
    int off_gt = my_gt ? atomicAdd(&cnt_gt, my_gt) : 0;
    int off_eq = my_eq ? atomicAdd(&cnt_eq, my_eq) : 0;
    __syncthreads();
    if (t == 0) {
        base_gt = cnt_gt ? (int)atomicAdd(&ctrl[0], (uint32_t)cnt_gt) : 0;
        base_eq = cnt_eq ? (int)atomicAdd(&ctrl[1], (uint32_t)cnt_eq) : 0;
    }
    __syncthreads();
    off_gt += base_gt;
    off_eq += base_eq;
    int2* __restrict__ crow = cand + (size_t)r * S_max;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int s = s0 + i * kChunkThreads + t;
        if (s >= s1) continue;
        const uint32_t dg = keys[i] >> 20;
        if (dg > d1) {
            orow[off_gt] = emit(s, wstart);
            if (osc) osc[off_gt] = v[i];
            ++off_gt;
        } else if (dg == d1) {
            crow[off_eq++] = make_int2((int)keys[i], s);
        }
    }
}

// Resolve the threshold bucket of each row among its (key, slot) candidates:
// the two remaining digits, from LDS when the candidates fit.
__global__ __launch_bounds__(kChunkThreads) void topk_resolve_kernel(
    const float* __restrict__ scores, int32_t S_max, const int32_t* __restrict__ positions, int32_t valid_len,
    int32_t k, int32_t window, uint32_t* __restrict__ ghist, const int2* __restrict__ cand,
    int32_t* __restrict__ out_idx, float* __restrict__ out_scores)
{
    __shared__ int hist[kBins];
    __shared__ int2 lcand[kResolveCap];
    __shared__ int wave_tot[kChunkThreads / 64];
    __shared__ int sh_digit, sh_above, cnt_gt, cnt_eq;

    const int r = blockIdx.x;
    // the threshold bin and the count above it, as the filter's chunk 0
    // found them, and the candidate count (the filter's running total);
    // read together with the position
    const uint32_t* __restrict__ ctrl = ghist + (size_t)r * kHeaderWords + kBins + kCoarse;
    const int n_cand = (int)ctrl[1];
    const uint32_t d1 = ctrl[2];
    const int above = (int)ctrl[3];
    const int nv = n_valid_of(positions, valid_len, r, S_max);
    if (nv <= k) return;  // uniform
    const int width = k + window;
    const int wstart = nv - window;
    const float* __restrict__ row = scores + (size_t)r * S_max;
    int32_t* __restrict__ orow = out_idx + (size_t)r * width;
    float* __restrict__ osc = out_scores ? out_scores + (size_t)r * k : nullptr;
    const int t = threadIdx.x;

    const bool in_lds = n_cand <= kResolveCap;
    const int2* __restrict__ crow = cand + (size_t)r * S_max;
    if (in_lds)
        for (int i = t; i < n_cand; i += kChunkThreads) lcand[i] = crow[i];
    __syncthreads();
    auto cand_at = [&](int i) -> int2 { return in_lds ? lcand[i] : crow[i]; };

    int remaining = k - above;
    uint32_t prefix = d1 << 20, pmask = 0xFFF00000u;
    if (remaining < n_cand) {
        const int shifts[2] = {8, 0};
        const int bits[2] = {12, 8};
        for (int pass = 0; pass < 2; ++pass) {
            const int nb = 1 << bits[pass];
            const int sh = shifts[pass];
            for (int i = t; i < nb; i += kChunkThreads) hist[i] = 0;
            __syncthreads();
            for (int i = t; i < n_cand; i += kChunkThreads) {
                const uint32_t key = (uint32_t)cand_at(i).x;
                if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & (nb - 1)], 1);
            }
            __syncthreads();
            find_bucket<kChunkThreads>(hist, nb, remaining, wave_tot, &sh_digit, &sh_above);
            const int d = sh_digit;
            remaining -= sh_above;
            prefix |= (uint32_t)d << sh;
            pmask |= (uint32_t)(nb - 1) << sh;
            const bool exact = hist[d] == remaining;
            __syncthreads();
            if (exact) break;
        }
    }
    if (t == 0) {
        cnt_gt = 0;
        cnt_eq = 0;
    }
    __syncthreads();
    const int n_gt = k - remaining;  // slots already placed or strictly above the final threshold
    for (int i = t; i < n_cand; i += kChunkThreads) {
        const int2 ck = cand_at(i);
        const uint32_t km = (uint32_t)ck.x & pmask;
        int pos = -1;
        if (km > prefix) {
            pos = above + atomicAdd(&cnt_gt, 1);
        } else if (km == prefix) {
            const int tk = atomicAdd(&cnt_eq, 1);
            if (tk < remaining) pos = n_gt + tk;
        }
        if (pos >= 0) {
            orow[pos] = emit(ck.y, wstart);
            if (osc) osc[pos] = row[ck.y];
        }
    }
}

bool use_chunked(int32_t M, int32_t S_max) { return S_max > kChunk && M < 1024; }

}  // namespace

size_t topk_workspace_bytes(int32_t M, int32_t S_max)
{
    if (!use_chunked(M, S_max)) return 0;
    return (size_t)M * kHeaderWords * sizeof(uint32_t) + (size_t)M * S_max * sizeof(int2);
}

size_t topk_header_words(int32_t M, int32_t S_max) { return use_chunked(M, S_max) ? (size_t)M * kHeaderWords : 0; }

hipError_t launch_topk(const float* scores, int32_t M, int32_t S_max, const int32_t* positions,
                       int32_t valid_len, int32_t k, int32_t window, int32_t* out_idx, float* out_scores,
                       void* workspace, bool header_zeroed, hipStream_t stream)
{
    if (!use_chunked(M, S_max)) {
        if (S_max <= kRowCap && (S_max & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0)
            topk_row_lds_kernel<<<M, kRowLdsThreads, 0, stream>>>(scores, S_max, positions, valid_len, k, window,
                                                                  out_idx, out_scores);
        else
            topk_row_kernel<<<M, kRowThreads, 0, stream>>>(scores, S_max, positions, valid_len, k, window, out_idx,
                                                           out_scores);
        return hipGetLastError();
    }
    uint32_t* ghist = static_cast<uint32_t*>(workspace);
    int2* cand = reinterpret_cast<int2*>(ghist + (size_t)M * kHeaderWords);
    const int n_words = M * kHeaderWords;
    if (!header_zeroed) topk_clear_kernel<<<(n_words + 255) / 256, 256, 0, stream>>>(ghist, n_words);
    // chunk size: 4096 slots, or 2048 when that would leave the chip short of workgroups
    if ((long long)M * ((S_max + kChunk - 1) / kChunk) < kSmallGridWgs) {
        const dim3 grid((S_max + kChunkSmall - 1) / kChunkSmall, M);
        topk_hist_kernel<kChunkSmall><<<grid, kChunkThreads, 0, stream>>>(scores, S_max, positions, valid_len, k, ghist);
        topk_filter_kernel<kChunkSmall><<<grid, kChunkThreads, 0, stream>>>(scores, S_max, positions, valid_len, k, window,
                                                                            ghist, cand, out_idx, out_scores);
    } else {
        const dim3 grid((S_max + kChunk - 1) / kChunk, M);
        topk_hist_kernel<kChunk><<<grid, kChunkThreads, 0, stream>>>(scores, S_max, positions, valid_len, k, ghist);
        topk_filter_kernel<kChunk><<<grid, kChunkThreads, 0, stream>>>(scores, S_max, positions, valid_len, k, window,
                                                                       ghist, cand, out_idx, out_scores);
    }
    topk_resolve_kernel<<<M, kChunkThreads, 0, stream>>>(scores, S_max, positions, valid_len, k, window, ghist, cand,
                                                         out_idx, out_scores);
    return hipGetLastError();
}

}  // namespace dsa
