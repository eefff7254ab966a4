// Decode lightning-indexer score (one query row per sequence) for gfx950.
//
// Definition (AWS Neuron "DeepSeek-V3.2 Sparse Indexer Kernel API
// Reference", Returns and Notes): every cached key slot s of row r gets
//   score = scale * sum_h w[r,h] * (q[r,h,:] . K[r,s,:])
// and slots the row cannot attend to get the finite mask bound.
//
// With the identity activation the head sum folds by linearity into one
// fp32 query, q_eff[d] = scale * sum_h w[r,h] q[r,h,d], so each slot costs
// one 128-long dot product: 0.5 flop per key byte, far below the HBM ridge.
// The kernel is therefore a coalesced streaming read of the key cache:
//   - grid (chunks of 512 slots, rows); chunks past n_valid only write the
//     mask bound, so the dispatcher balances rows of different lengths;
//   - bf16 keys: 16 lanes x 16 B cover one 256-B slot, a wave load moves
//     4 consecutive slots (1 KiB); fp8 keys: 8 lanes x 16 B per 128-B slot;
//   - the first key loads are issued before the fold so their latency
//     overlaps it; loads are double-buffered in registers;
//   - partial dots are summed across the lanes of a slot with DPP row ops;
//   - a chunk's scores are staged in LDS and written with 16-byte
//     non-temporal stores: scattered 4-byte score stores interleaved with
//     the key stream cost ~10% of the bandwidth;
//   - paged caches (a block table maps each page-sized run of a sequence's
//     slots to a page of a shared pool, pages a power of two >= 64 slots):
//     a wave's 64 consecutive slots of one load round never straddle a page,
//     so one table lookup per round gives their rows.
#include "device_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 512;      // slots per workgroup
constexpr int kUnrollBf16 = 16;  // loads in flight per lane per buffer (bf16: 64 slots per wave)
constexpr int kUnrollFp8 = 8;    // (fp8: 64 slots per wave)

// q_eff[d] = scale * sum_h w[h] q[h][d] into LDS (256 threads: 16 head
// groups x 16 blocks of 8 dims).
__device__ __forceinline__ void fold_query(const uint16_t* __restrict__ q, const float* __restrict__ w, int H,
                                           float scale, float* red, float* qe)
{
    const int t = threadIdx.x;
    const int dblk = t & 15;
    const int hg = t >> 4;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    // the first 64 heads: all loads issued before the first use (heads past H
    // read head 0 with weight 0), so they cost one memory latency, not four
    {
        u32x4 v[4];
        float wh[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int h = hg + 16 * u;
            const int hc = h < H ? h : 0;
            v[u] = *reinterpret_cast<const u32x4*>(q + (size_t)hc * 128 + dblk * 8);
            wh[u] = w[hc];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float f = hg + 16 * u < H ? wh[u] : 0.f;
            acc[0] = fmaf(f, bf16_lo(v[u].x), acc[0]);
            acc[1] = fmaf(f, bf16_hi(v[u].x), acc[1]);
            acc[2] = fmaf(f, bf16_lo(v[u].y), acc[2]);
            acc[3] = fmaf(f, bf16_hi(v[u].y), acc[3]);
            acc[4] = fmaf(f, bf16_lo(v[u].z), acc[4]);
            acc[5] = fmaf(f, bf16_hi(v[u].z), acc[5]);
            acc[6] = fmaf(f, bf16_lo(v[u].w), acc[6]);
            acc[7] = fmaf(f, bf16_hi(v[u].w), acc[7]);
        }
    }
    for (int h = hg + 64; h < H; h += 16) {  // heads 64 .. 127
        const u32x4 v = *reinterpret_cast<const u32x4*>(q + (size_t)h * 128 + dblk * 8);
        const float wh = w[h];
        acc[0] = fmaf(wh, bf16_lo(v.x), acc[0]);
        acc[1] = fmaf(wh, bf16_hi(v.x), acc[1]);
        acc[2] = fmaf(wh, bf16_lo(v.y), acc[2]);
        acc[3] = fmaf(wh, bf16_hi(v.y), acc[3]);
        acc[4] = fmaf(wh, bf16_lo(v.z), acc[4]);
        acc[5] = fmaf(wh, bf16_hi(v.z), acc[5]);
        acc[6] = fmaf(wh, bf16_lo(v.w), acc[6]);
        acc[7] = fmaf(wh, bf16_hi(v.w), acc[7]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) red[hg * 128 + dblk * 8 + i] = acc[i];
    __syncthreads();
    if (t < 128) {
        float s = 0.f;
#pragma unroll
        for (int g = 0; g < 16; ++g) s += red[g * 128 + t];
        qe[t] = s * scale;
    }
    __syncthreads();
}

// Write a chunk's staged scores [s0, se) to out: 16-byte non-temporal
// stores when the chunk is full and aligned.
__device__ __forceinline__ void flush_stage(const float* stage, float* __restrict__ out, int s0, int se)
{
    __syncthreads();
    if (se - s0 == kChunk && (reinterpret_cast<uintptr_t>(out + s0) & 15) == 0) {
        for (int i = threadIdx.x; i < kChunk / 4; i += kThreads)
            __builtin_nontemporal_store(reinterpret_cast<const u32x4*>(stage)[i],
                                        reinterpret_cast<u32x4*>(out + s0) + i);
    } else {
        for (int i = threadIdx.x; i < se - s0; i += kThreads) out[s0 + i] = stage[i];
    }
}

__device__ __forceinline__ float dot8_bf16(const float* qv, u32x4 v)
{
    float p = qv[0] * bf16_lo(v.x);
    p = fmaf(qv[1], bf16_hi(v.x), p);
    p = fmaf(qv[2], bf16_lo(v.y), p);
    p = fmaf(qv[3], bf16_hi(v.y), p);
    p = fmaf(qv[4], bf16_lo(v.z), p);
    p = fmaf(qv[5], bf16_hi(v.z), p);
    p = fmaf(qv[6], bf16_lo(v.w), p);
    p = fmaf(qv[7], bf16_hi(v.w), p);
    return p;
}

// bf16 keys: slot = 256 B = 16 lanes x 16 B.  Per wave and buffer:
// kUnroll x 4 consecutive slots.
template <bool PAGED>
__global__ __launch_bounds__(kThreads) void score_decode_bf16_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ k,
    const int32_t* __restrict__ positions, int32_t valid_len, int32_t H, int32_t S_max, float scale,
    float* __restrict__ scores, uint32_t* __restrict__ zero_ptr, size_t zero_words, PageMap pm)
{
    clear_words(zero_ptr, zero_words);
    constexpr int kUnroll = kUnrollBf16;
    __shared__ float red[16 * 128];
    __shared__ float qe[128];
    __shared__ __attribute__((aligned(16))) float stage[kChunk];
    const int r = blockIdx.y;
    const int s0 = blockIdx.x * kChunk;
    const int s1 = min(s0 + kChunk, S_max);
    const int nv = n_valid_of(positions, valid_len, r, S_max);
    float* __restrict__ out = scores + (size_t)r * S_max;

    const float mb = mask_bound();
    for (int s = max(s0, nv) + (int)threadIdx.x; s < s1; s += kThreads) out[s] = mb;
    const int se = min(s1, nv);
    if (s0 >= se) return;  // uniform over the workgroup

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;      // slot within a group of 4
    const int dblk = lane & 15;   // dims 8*dblk .. 8*dblk+7
    constexpr int kWaveSlots = 4 * kUnroll;
    constexpr int kIterSlots = 4 * kWaveSlots;
    // keys of the wave's slots [base, base + 64) start at row store_row(base).
    // Paged, the rows of the next round are looked up one round ahead (the
    // table read is a dependent load in front of that round's key loads).
    auto round_keys = [&](const int base) {
        return k + store_row<PAGED>(pm, r, base, S_max) * 128 + dblk * 8;
    };

    u32x4 buf[kUnroll];
    int base = s0 + wave * kWaveSlots;
    const uint16_t* __restrict__ kr_next = round_keys(base + kIterSlots);
    {
        const uint16_t* __restrict__ kr = round_keys(base);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int s = base + 4 * u + g;
            buf[u] = (s < se) ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kr + (size_t)(4 * u + g) * 128))
                              : u32x4{0, 0, 0, 0};
        }
    }

    fold_query(q + (size_t)r * H * 128, w + (size_t)r * H, H, scale, red, qe);
    float qv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[i] = qe[dblk * 8 + i];

    for (; base < se; base += kIterSlots) {
        u32x4 cur[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) cur[u] = buf[u];
        const int nb = base + kIterSlots;
        if (nb < se) {
            const uint16_t* __restrict__ kr = kr_next;
            kr_next = round_keys(nb + kIterSlots);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int s = nb + 4 * u + g;
                buf[u] = (s < se) ? __builtin_nontemporal_load(
                                        reinterpret_cast<const u32x4*>(kr + (size_t)(4 * u + g) * 128))
                                  : u32x4{0, 0, 0, 0};
            }
        }
        float part[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) part[u] = row16_sum(dot8_bf16(qv, cur[u]));
        // lane (g, j) stages slot base + 4j + g (all 16 lanes of a group)
        float val = part[0];
#pragma unroll
        for (int u = 1; u < kUnroll; ++u) val = (dblk == u) ? part[u] : val;
        const int s = base + 4 * dblk + g;
        if (dblk < kUnroll && s < se) stage[s - s0] = val;
    }
    flush_stage(stage, out, s0, se);
}

// fp8 keys: slot = 128 B codes + one fp32 scale; 8 lanes x 16 B per slot,
// a wave load moves 8 consecutive slots.
__device__ __forceinline__ float dot16_fp8(const float* qv, u32x4 v)
{
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
    float p = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[i], false);
        const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[i], true);
        p = fmaf(qv[4 * i + 0], a[0], p);
        p = fmaf(qv[4 * i + 1], a[1], p);
        p = fmaf(qv[4 * i + 2], b[0], p);
        p = fmaf(qv[4 * i + 3], b[1], p);
    }
    return p;
}

template <bool PAGED>
__global__ __launch_bounds__(kThreads) void score_decode_fp8_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint8_t* __restrict__ k,
    const float* __restrict__ k_scale, const int32_t* __restrict__ positions, int32_t valid_len, int32_t H,
    int32_t S_max, float scale, float* __restrict__ scores, uint32_t* __restrict__ zero_ptr, size_t zero_words,
    PageMap pm)
{
    clear_words(zero_ptr, zero_words);
    constexpr int kUnroll = kUnrollFp8;
    __shared__ float red[16 * 128];
    __shared__ float qe[128];
    __shared__ __attribute__((aligned(16))) float stage[kChunk];
    const int r = blockIdx.y;
    const int s0 = blockIdx.x * kChunk;
    const int s1 = min(s0 + kChunk, S_max);
    const int nv = n_valid_of(positions, valid_len, r, S_max);
    float* __restrict__ out = scores + (size_t)r * S_max;

    const float mb = mask_bound();
    for (int s = max(s0, nv) + (int)threadIdx.x; s < s1; s += kThreads) out[s] = mb;
    const int se = min(s1, nv);
    if (s0 >= se) return;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 3;     // slot within a group of 8
    const int dblk = lane & 7;   // dims 16*dblk .. 16*dblk+15
    constexpr int kWaveSlots = 8 * kUnroll;
    constexpr int kIterSlots = 4 * kWaveSlots;

    // codes and scales of the wave's slots [base, base + 64) start at row store_row(base)
    u32x4 buf[kUnroll];
    float sbuf;
    int base = s0 + wave * kWaveSlots;
    size_t row_next = store_row<PAGED>(pm, r, base + kIterSlots, S_max);  // next round's rows, looked up ahead
    auto load_round = [&](const int b0, const size_t row0) {
        const uint8_t* __restrict__ kr = k + row0 * 128 + dblk * 16;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int s = b0 + 8 * u + g;
            buf[u] = (s < se) ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kr + (size_t)(8 * u + g) * 128))
                              : u32x4{0, 0, 0, 0};
        }
        const int s = b0 + 8 * dblk + g;
        sbuf = (s < se) ? k_scale[row0 + 8 * dblk + g] : 0.f;
    };
    load_round(base, store_row<PAGED>(pm, r, base, S_max));

    fold_query(q + (size_t)r * H * 128, w + (size_t)r * H, H, scale, red, qe);
    float qv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) qv[i] = qe[dblk * 16 + i];

    for (; base < se; base += kIterSlots) {
        u32x4 cur[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) cur[u] = buf[u];
        const float cs = sbuf;
        const int nb = base + kIterSlots;
        if (nb < se) {
            const size_t row0 = row_next;
            row_next = store_row<PAGED>(pm, r, nb + kIterSlots, S_max);
            load_round(nb, row0);
        }
        float part[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) part[u] = row8_sum(dot16_fp8(qv, cur[u]));
        float val = part[0];
#pragma unroll
        for (int u = 1; u < kUnroll; ++u) val = (dblk == u) ? part[u] : val;
        const int s = base + 8 * dblk + g;
        if (s < se) stage[s - s0] = val * cs;
    }
    flush_stage(stage, out, s0, se);
}

}  // namespace

hipError_t launch_score_decode(const void* q, const float* w, const void* k_cache, const float* k_scale,
                               bool key_fp8, const int32_t* positions, int32_t valid_len, int32_t M,
                               int32_t H, int32_t S_max, float scale, float* scores, uint32_t* zero_ptr,
                               size_t zero_words, const PageMap* paging, hipStream_t stream)
{
    const dim3 grid((S_max + kChunk - 1) / kChunk, M);
    const PageMap pm = paging ? *paging : PageMap{nullptr, 0, 0, 0};
    const auto* qq = static_cast<const uint16_t*>(q);
    if (key_fp8) {
        const auto* kc = static_cast<const uint8_t*>(k_cache);
        if (paging)
            score_decode_fp8_kernel<true><<<grid, kThreads, 0, stream>>>(qq, w, kc, k_scale, positions, valid_len, H,
                                                                         S_max, scale, scores, zero_ptr, zero_words, pm);
        else
            score_decode_fp8_kernel<false><<<grid, kThreads, 0, stream>>>(qq, w, kc, k_scale, positions, valid_len, H,
                                                                          S_max, scale, scores, zero_ptr, zero_words, pm);
    } else {
        const auto* kc = static_cast<const uint16_t*>(k_cache);
        if (paging)
            score_decode_bf16_kernel<true><<<grid, kThreads, 0, stream>>>(qq, w, kc, positions, valid_len, H, S_max,
                                                                          scale, scores, zero_ptr, zero_words, pm);
        else
            score_decode_bf16_kernel<false><<<grid, kThreads, 0, stream>>>(qq, w, kc, positions, valid_len, H, S_max,
                                                                           scale, scores, zero_ptr, zero_words, pm);
    }
    return hipGetLastError();
}

}  // namespace dsa
