// Top-k slot selection per score row for gfx950.
//
// Contract (AWS Neuron "DeepSeek-V3.2 Sparse Indexer Kernel API
// Reference", Returns and Notes): the index_topk highest-scoring attendable
// slots of each row, as an unordered set, padded with -1 when a row has
// fewer attendable slots.
//
// Radix select on order-preserving 32-bit keys of the fp32 scores, one
// 1024-thread workgroup per row, histograms in LDS:
//   pass 1: 12-bit digit (key bits 31..20) over all attendable slots;
//   pass 2: 12-bit digit (19..8) over keys in the selected bucket;
//   pass 3: 8-bit digit (7..0);
// after each pass the bucket holding the k-th largest key is found by a
// suffix scan of the histogram; if the bucket's count equals what is still
// needed the threshold is final.  A last pass writes every key above the
// threshold bucket and the first `remaining` keys inside it (ties at the
// boundary are resolved by arrival order, which the set contract allows).
//
// The decode step uses the same kernel to emit its index list: with
// window > 0 a selected slot inside the window [n_valid - window, n_valid)
// is written as -1 and the window positions follow the top-k columns.
#include "device_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxBins = 4096;

// Inclusive prefix sum over the workgroup (1024 threads).
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

// Find digit d with  above(d) < need <= above(d) + hist[d], where above(d) is
// the count of keys with digit > d.  Writes d and above(d) to shared memory.
__device__ void find_bucket(const int* hist, int nbins, int need, int* wave_tot, int* res_digit, int* res_above)
{
    const int per = nbins / kThreads > 0 ? nbins / kThreads : 1;
    // thread t owns bins [hi_bin - per + 1, hi_bin], counted from the top
    const int t = threadIdx.x;
    const int top = nbins - 1 - t * per;  // highest bin of this thread
    int local = 0;
    if (top >= 0)
        for (int i = 0; i < per; ++i) local += hist[top - i];
    const int incl = block_inclusive_scan(local, wave_tot);  // keys in bins > top - per
    const int excl = incl - local;                            // keys in bins > top
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

__global__ __launch_bounds__(kThreads) void topk_radix_kernel(
    const float* __restrict__ scores, int32_t S_max, const int32_t* __restrict__ positions, int32_t valid_len,
    int32_t k, int32_t window, int32_t* __restrict__ out_idx, float* __restrict__ out_scores)
{
    __shared__ int hist[kMaxBins];
    __shared__ int wave_tot[kWaves];
    __shared__ int sh_digit, sh_above, cnt_gt, cnt_eq;

    const int r = blockIdx.x;
    const int nv = n_valid_of(positions, valid_len, r, S_max);
    const int width = k + window;
    const int wstart = nv - window;
    const float* __restrict__ row = scores + (size_t)r * S_max;
    int32_t* __restrict__ orow = out_idx + (size_t)r * width;
    float* __restrict__ osc = out_scores ? out_scores + (size_t)r * k : nullptr;
    const int t = threadIdx.x;

    for (int i = t; i < window; i += kThreads) {
        const int p = wstart + i;
        orow[k + i] = p < 0 ? -1 : p;
    }

    if (nv <= k) {
        for (int j = t; j < k; j += kThreads) {
            const int s = j < nv ? j : -1;
            orow[j] = (s >= wstart) ? -1 : s;
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
        for (int i = t; i < nb; i += kThreads) hist[i] = 0;
        __syncthreads();
        for (int s = t; s < nv; s += kThreads) {
            const uint32_t key = f32_order_key(row[s]);
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & (nb - 1)], 1);
        }
        __syncthreads();
        find_bucket(hist, nb, remaining, wave_tot, &sh_digit, &sh_above);
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
    for (int s = t; s < nv; s += kThreads) {
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
            orow[pos] = (s >= wstart) ? -1 : s;
            if (osc) osc[pos] = v;
        }
    }
}

}  // namespace

hipError_t launch_topk(const float* scores, int32_t M, int32_t S_max, const int32_t* positions,
                       int32_t valid_len, int32_t k, int32_t window, int32_t* out_idx, float* out_scores,
                       hipStream_t stream)
{
    topk_radix_kernel<<<M, kThreads, 0, stream>>>(scores, S_max, positions, valid_len, k, window, out_idx,
                                                  out_scores);
    return hipGetLastError();
}

}  // namespace dsa
