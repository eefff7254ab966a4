// Prefill lightning-indexer score with the identity activation, for gfx950.
//
// Definition (AWS Neuron "Sparse Attention Indexer MX BF16Score Kernel API
// Reference", :return: and Dimensions; "DeepSeek-V3.2 Sparse Indexer Kernel
// API Reference", Returns and Notes): for query row r and key slot
// s < n_valid(r)
//   score[r, s] = scale * sum_h w[r, h] * (q[r, h, :] . K[s, :])
// and the finite mask bound elsewhere.
//
// With the identity activation the head sum folds by linearity into one
// query per row, q_eff = scale * sum_h w[r, h] q[r, h, :] (fp32), exactly as
// in the decode scorer.  The fold cuts the contraction from 64 heads x 128
// dims to 128 dims per (row, key) pair, so this kernel is bound by writing
// the score matrix, not by MFMA:
//   * workgroup = two 16-row tiles of one sequence, tile a and tile
//     n - 1 - a of its n tiles, so every workgroup has about the same causal
//     work (one tile's rows see few keys, the other's many); 8 waves, two per
//     SIMD; the prologue folds each row's q in fp32 (lane = 8 dims of every fourth head, 16-byte
//     loads, two rows = 32 loads in flight per lane, the four head groups
//     summed with lane swaps) and splits q_eff into bf16 hi + lo parts
//     (q_eff - hi rounded again), which keeps 16 significant bits of it, far
//     below the score tolerance;
//   * v_mfma_f32_32x32x16_bf16 with M = 32 = 16 rows x {hi, lo}, N = 32 keys,
//     K = 16 dims: the A operands (2 row tiles x 8 K steps) stay in
//     registers; lane (key n, half g) of the accumulator holds rows
//     8 (j / 4) + 4 g + j % 4, so the hi and lo results of a query row sit in
//     the same lane (j and j + 8) and add up without lane exchange;
//   * key tiles of 32 keys are dealt to the 8 waves round-robin; the B
//     operands come straight from memory (a sequence's keys stay in L2),
//     one tile ahead;
//   * a row tile whose rows are all past their causal limit in a key tile
//     skips its MFMAs and only writes the mask bound;
//   * q (read once) and the score matrix (written once) stream with
//     non-temporal loads and stores, so they do not displace the keys in
//     L2: with plain ones the q fold read at ~3.1 TB/s and the kernel took
//     144 us at 8192 x 8192, against 22 us for the fold and 108 us.  The
//     score stores also carry device scope (sc1): 97 against 99.5 us, the
//     scores bit-equal; plain or sc0 stores took 121-125 us.
#include "device_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kRows = 32;  // query rows per workgroup: two tiles of 16
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kKeys = 32;  // keys per tile
constexpr int kSteps = 8;  // K steps of 16 dims
constexpr int kBufferWord3 = 0x00020000;  // buffer descriptor word 3: 32-bit data, raw (byte-addressed) access
constexpr int kStoreNt = 18;              // buffer store cache policy: non-temporal, device scope (nt sc1)

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

__device__ __forceinline__ uint32_t bf16_bits(float f) { return f32_to_bf16_bits(f); }

// sum over the 4 lane groups (lanes l, l + 16, l + 32, l + 48)
__device__ __forceinline__ float lane_group_sum(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__global__ __launch_bounds__(kThreads) void score_prefill_fold_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ k,
    const int32_t* __restrict__ positions, int32_t valid_len, int32_t rows_per_seq, int32_t H, int32_t S_max,
    float scale, float* __restrict__ scores)
{
    // folded queries: row i, part p (0 = hi, 1 = lo), 128 dims of bf16
    __shared__ __attribute__((aligned(16))) uint16_t qf[kRows][2][128];
    __shared__ int nv_sh[kRows];
    __shared__ float w_sh[kRows][64];  // per-head weights of the first 64 heads of each row

    // row tiles a and nt - 1 - a of the sequence (the middle tile of an odd
    // count pairs with nothing)
    const int nt = (rows_per_seq + 15) / 16;
    const int wg_per_seq = (nt + 1) / 2;
    const int seq = blockIdx.x / wg_per_seq;
    const int a = blockIdx.x - seq * wg_per_seq;
    const int tile_m[2] = {a, nt - 1 - a};
    int base_m[2], cnt_m[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const bool used = m == 0 || tile_m[1] != a;
        base_m[m] = seq * rows_per_seq + 16 * tile_m[m];
        cnt_m[m] = used ? min(16, rows_per_seq - 16 * tile_m[m]) : 0;
    }
    // workgroup row i (0..31) = row i & 15 of tile i >> 4
    auto row_ok = [&](int i) { return (i & 15) < cnt_m[i >> 4]; };
    auto grow = [&](int i) { return base_m[i >> 4] + (i & 15); };
    const uint16_t* __restrict__ ks = k + (size_t)seq * S_max * 128;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // the rows' first 64 head weights, with coalesced loads
    for (int x = threadIdx.x; x < kRows * 64; x += kThreads) {
        const int i = x >> 6, h = x & 63;
        w_sh[i][h] = (row_ok(i) && h < H) ? w[(size_t)grow(i) * H + h] : 0.f;
    }
    __syncthreads();

    // ---- fold: wave w folds rows 4 w .. 4 w + 3, two at a time; lane (head
    // group hq, dim block db) accumulates dims 8 db .. 8 db + 7 of heads
    // 4 u + hq, then the four head groups are summed
    {
        const int hq = lane >> 4;
        const int db = lane & 15;
        for (int i0 = 4 * wave; i0 < 4 * wave + 4; i0 += 2) {
            u32x4 v[2][16];
            float wv[2][16];
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const int i = i0 + rr;
                const int r = row_ok(i) ? grow(i) : base_m[0];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int h = 4 * u + hq;
                    const bool ok = row_ok(i) && h < H;
                    v[rr][u] = ok ? __builtin_nontemporal_load(
                                        reinterpret_cast<const u32x4*>(q + ((size_t)r * H + h) * 128 + 8 * db))
                                  : u32x4{0u, 0u, 0u, 0u};
                    wv[rr][u] = w_sh[i][4 * u + hq];  // 0 for rows and heads out of range
                }
            }
            float acc[2][8];
#pragma unroll
            for (int rr = 0; rr < 2; ++rr)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[rr][e] = 0.f;
#pragma unroll
            for (int rr = 0; rr < 2; ++rr)
#pragma unroll
                for (int u = 0; u < 16; ++u)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[rr][2 * e] = fmaf(wv[rr][u], bf16_lo(v[rr][u][e]), acc[rr][2 * e]);
                        acc[rr][2 * e + 1] = fmaf(wv[rr][u], bf16_hi(v[rr][u][e]), acc[rr][2 * e + 1]);
                    }
            // heads beyond 64 (H up to 128): a second pass over the same lanes
            for (int h0 = 64; h0 < H; h0 += 64) {
#pragma unroll
                for (int rr = 0; rr < 2; ++rr) {
                    const int i = i0 + rr;
                    const int r = row_ok(i) ? grow(i) : base_m[0];
#pragma unroll
                    for (int u = 0; u < 16; ++u) {
                        const int h = h0 + 4 * u + hq;
                        if (row_ok(i) && h < H) {
                            const u32x4 x = *reinterpret_cast<const u32x4*>(q + ((size_t)r * H + h) * 128 + 8 * db);
                            const float wh = w[(size_t)r * H + h];
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                acc[rr][2 * e] = fmaf(wh, bf16_lo(x[e]), acc[rr][2 * e]);
                                acc[rr][2 * e + 1] = fmaf(wh, bf16_hi(x[e]), acc[rr][2 * e + 1]);
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x0 = lane_group_sum(acc[rr][2 * e]) * scale;
                    const float x1 = lane_group_sum(acc[rr][2 * e + 1]) * scale;
                    const uint32_t b0 = bf16_bits(x0), b1 = bf16_bits(x1);
                    hi[e] = b0 | (b1 << 16);
                    lo[e] = bf16_bits(x0 - __uint_as_float(b0 << 16)) | (bf16_bits(x1 - __uint_as_float(b1 << 16)) << 16);
                }
                if (hq == 0) {
                    *reinterpret_cast<u32x4*>(&qf[i0 + rr][0][8 * db]) = u32x4{hi[0], hi[1], hi[2], hi[3]};
                    *reinterpret_cast<u32x4*>(&qf[i0 + rr][1][8 * db]) = u32x4{lo[0], lo[1], lo[2], lo[3]};
                }
            }
        }
    }
    if (threadIdx.x < kRows)
        nv_sh[threadIdx.x] = row_ok(threadIdx.x) ? n_valid_of(positions, valid_len, grow(threadIdx.x), S_max) : 0;
    __syncthreads();

    // ---- A operands: row tile m (query rows 16 m .. 16 m + 15), K step t; lane
    // (A row i = lane % 32, half g = lane / 32): i < 16 -> hi of row 16 m + i,
    // i >= 16 -> lo of row 16 m + i - 16; dims 16 t + 8 g .. + 7
    const int n = lane & 31;
    const int g = lane >> 5;
    u32x4 qa[2][kSteps];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int t = 0; t < kSteps; ++t)
            qa[m][t] = *reinterpret_cast<const u32x4*>(&qf[16 * m + (n & 15)][n >> 4][16 * t + 8 * g]);
    // this lane's query rows per row tile: 8 (j / 4) + 4 g + j % 4, j < 8
    int nv_r[2][8];
    int max_nv_m[2] = {0, 0};
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int j = 0; j < 8; ++j) nv_r[m][j] = nv_sh[16 * m + 8 * (j / 4) + 4 * g + j % 4];
    for (int i = 0; i < kRows; ++i) max_nv_m[i >> 4] = max(max_nv_m[i >> 4], nv_sh[i]);
    const int max_nv = max(max_nv_m[0], max_nv_m[1]);
    const float mb = mask_bound();

    // Score rows of the two row tiles as buffers.  A store for a row past the
    // tile's rows or a key past S_max gets an offset beyond the buffer bound,
    // which the hardware drops: every store is issued unconditionally, so the
    // compiler can count them and wait for the next key tile's loads alone
    // (loads and stores share one in-order counter here) instead of draining
    // the previous tile's score stores on every tile.
    __amdgpu_buffer_rsrc_t srs[2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
        srs[m] = __builtin_amdgcn_make_buffer_rsrc((void*)(scores + (size_t)base_m[m] * S_max), 0,
                                                   cnt_m[m] * S_max * 4, kBufferWord3);
    auto store = [&](int m, int j, int s, float v) {
        const int rl = 8 * (j / 4) + 4 * g + j % 4;  // row of tile m
        const uint32_t off = (rl < cnt_m[m] && s < S_max) ? (uint32_t)(rl * S_max + s) * 4u : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), srs[m], off, 0, kStoreNt);
    };

    const int ntiles = (S_max + kKeys - 1) / kKeys;
    auto load_tile = [&](int kt, u32x4 (&b)[kSteps]) {
        const int s = kt * kKeys + n;
        const uint16_t* kp = ks + (size_t)(s < S_max ? s : 0) * 128 + 8 * g;
#pragma unroll
        for (int t = 0; t < kSteps; ++t) b[t] = *reinterpret_cast<const u32x4*>(kp + 16 * t);
    };
    // key tiles holding a live slot of some row of the workgroup: wave w takes
    // tiles w, w + kWaves, ...; each iteration loads the wave's next tile (the
    // last one again at the end, so every iteration issues the same loads)
    const int n_live = min(ntiles, (max_nv + kKeys - 1) / kKeys);
    int kt = wave;
    if (kt < n_live) {
        u32x4 bcur[kSteps];
        load_tile(kt, bcur);
        // stores past every buffer bound (dropped): each iteration then starts
        // with the same pending operations, the next tile's loads followed by a
        // tile's 16 stores, so the wait for the loads leaves the stores in flight
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int j = 0; j < 8; ++j) __builtin_amdgcn_raw_buffer_store_b32(0u, srs[m], 0x80000000u, 0, kStoreNt);
        for (; kt < n_live; kt += kWaves) {
            const int s = kt * kKeys + n;
            u32x4 b[kSteps];
#pragma unroll
            for (int t = 0; t < kSteps; ++t) b[t] = bcur[t];
            load_tile(min(kt + kWaves, n_live - 1), bcur);  // the next tile, one ahead
            f32x16 c[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                c[m] = f32x16{};
                if (kt * kKeys < max_nv_m[m])  // uniform: skip a row tile that is all masked here
#pragma unroll
                    for (int t = 0; t < kSteps; ++t) c[m] = mfma32(qa[m][t], b[t], c[m]);
            }
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int j = 0; j < 8; ++j) store(m, j, s, s < nv_r[m][j] ? c[m][j] + c[m][j + 8] : mb);
        }
    }
    // tiles past every row's causal limit: the mask bound only
    for (kt = n_live + ((wave - n_live) % kWaves + kWaves) % kWaves; kt < ntiles; kt += kWaves) {
        const int s = kt * kKeys + n;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int j = 0; j < 8; ++j) store(m, j, s, mb);
    }
}

}  // namespace

hipError_t launch_score_prefill_fold(const void* q, const float* w, const void* k_cache, const int32_t* positions,
                                     int32_t valid_len, int32_t M, int32_t rows_per_seq, int32_t H, int32_t S_max,
                                     float scale, float* scores, hipStream_t stream)
{
    const int n_seq = M / rows_per_seq;
    const int wg_per_seq = ((rows_per_seq + 15) / 16 + 1) / 2;
    score_prefill_fold_kernel<<<n_seq * wg_per_seq, kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(q), w, static_cast<const uint16_t*>(k_cache), positions, valid_len,
        rows_per_seq, H, S_max, scale, scores);
    return hipGetLastError();
}

}  // namespace dsa

