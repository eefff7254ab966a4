// Prefill lightning-indexer score for gfx950: rows_per_seq query rows share
// one key cache and each row attends causally.
//
// Definition (AWS Neuron "Sparse Attention Indexer MX BF16Score Kernel API
// Reference", :return: and Dimensions -- pre-top-k per-position scores over
// [0, end_pos), end_pos = start_pos + S; Notes -- the score matmul runs in
// bf16): for row r and slot s < n_valid(r)
//   score[r, s] = scale * sum_h w[r, h] * phi( q[r, h, :] . K[s, :] )
// and the mask bound elsewhere.
//
// This is a dense per-head contraction, so it runs on MFMA:
//   * workgroup = 8 consecutive query rows of one sequence, one per wave
//     (2 waves per SIMD); groups with the longest causal range go first;
//   * v_mfma_f32_32x32x16_bf16 with M = 32 heads, N = 32 keys, K = 16 dims:
//     each wave keeps its row's q (64 heads x 128 dims) in registers as the
//     A operand for the whole key loop (2 head tiles x 8 K steps);
//   * the B operand, a 32-key tile of K (8 KiB), is copied HBM/L2 -> LDS with
//     16-byte global_load_lds into two distinct, double-buffered LDS arrays
//     (rows padded to 17 x 16 B so operand reads avoid bank conflicts) and
//     shared by the 8 waves;
//   * epilogue in registers: each lane holds 16 heads of one key per head
//     tile (accumulator row = 8 (j / 4) + 4 (lane / 32) + j % 4, column =
//     lane % 32); it applies phi, weights by w[r, h] (held in registers),
//     sums, adds the other lane half and scales;
//   * tiles past a row's causal limit are skipped (the workgroup stops at its
//     last row's limit); the rest of the row gets the mask bound with 16-byte
//     stores.
// The identity-phi fold used for decode (one pre-summed query per row) is
// not used here: on bf16 MFMA it would round the folded query to bf16, and
// it does not exist for phi = ReLU.
#include "device_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kQ = 8;        // query rows (waves) per workgroup
constexpr int kThreads = 64 * kQ;
constexpr int kTile = 32;    // keys per tile
constexpr int kRowU = 17;    // padded key row: 16 data units of 16 B + 1 pad
constexpr int kTileU = kTile * kRowU;

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__global__ __launch_bounds__(kThreads, 1) void score_prefill_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ k,
    const int32_t* __restrict__ positions, int32_t valid_len, int32_t rows_per_seq, int32_t H, int32_t S_max,
    float scale, int32_t relu, float* __restrict__ scores)
{
    __shared__ __attribute__((aligned(16))) u32x4 kt0[kTileU];
    __shared__ __attribute__((aligned(16))) u32x4 kt1[kTileU];
    __shared__ int s_nv[kQ];

    const int groups_per_seq = (rows_per_seq + kQ - 1) / kQ;
    const int gid = (int)(gridDim.x - 1 - blockIdx.x);  // late (long) groups first
    const int seq = gid / groups_per_seq;
    const int grp = gid - seq * groups_per_seq;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int qi = grp * kQ + wave;
    const bool q_ok = qi < rows_per_seq;
    const size_t r = (size_t)seq * rows_per_seq + (q_ok ? qi : 0);
    const int nv = q_ok ? n_valid_of(positions, valid_len, (int32_t)r, S_max) : 0;
    const int m = lane & 31;   // accumulator column: key within the tile; A row: head within the tile
    const int g = lane >> 5;   // lane half
    const uint16_t* __restrict__ kseq = k + (size_t)seq * S_max * 128;

    if (lane == 0) s_nv[wave] = nv;

    // A operand: q[r][32 mt + m][16 t + 8 g .. +7]
    u32x4 qa[2][8];
    float wv[2][16];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const int h = 32 * mt + m;
        const bool h_ok = q_ok && h < H;
        const uint16_t* qh = q + (r * H + (h_ok ? h : 0)) * 128 + 8 * g;
#pragma unroll
        for (int t = 0; t < 8; ++t)
            qa[mt][t] = h_ok ? *reinterpret_cast<const u32x4*>(qh + 16 * t) : u32x4{0, 0, 0, 0};
        // weights of the heads this lane accumulates: 32 mt + 8 jj + 4 g + i
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int hh = 32 * mt + 8 * jj + 4 * g + i;
                wv[mt][4 * jj + i] = (q_ok && hh < H) ? w[r * H + hh] : 0.f;
            }
    }
    __syncthreads();
    int nv_max = 0;
#pragma unroll
    for (int i = 0; i < kQ; ++i) nv_max = max(nv_max, s_nv[i]);
    const int ntiles = (nv_max + kTile - 1) / kTile;

    // LDS DMA of key tile `tile` into dst (waves 0..7 cover units 0..511, wave 0 the last 32)
    auto load_tile = [&](int tile, u32x4* dst) {
        for (int u0 = 0; u0 < kTileU; u0 += kThreads) {
            const int ub = u0 + 64 * wave_u;  // wave-uniform
            if (ub < kTileU) {
                const int u = ub + lane;
                const int kk = u / kRowU;
                int ch = u - kk * kRowU;
                ch = ch < 16 ? ch : 0;  // pad unit: any valid address
                int s = tile * kTile + kk;
                s = s < S_max ? s : S_max - 1;
                if (u < kTileU)
                    __builtin_amdgcn_global_load_lds(kseq + (size_t)s * 128 + 8 * ch, (lds_void*)(dst + ub), 16, 0, 0);
            }
        }
    };

    const float mb = mask_bound();
    float* __restrict__ out = scores + r * S_max;
    auto run_tile = [&](const int tile, const u32x4* kb, u32x4* nb) {
        wait_vmem();
        __syncthreads();  // tile resident for all waves; everyone finished the previous tile
        if (tile + 1 < ntiles) load_tile(tile + 1, nb);
        f32x16 c0 = {}, c1 = {};
        const u32x4* kr = kb + m * kRowU + g;
        u32x4 b = kr[0];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const u32x4 bn = (t + 1 < 8) ? kr[2 * (t + 1)] : b;
            c0 = mfma32(qa[0][t], b, c0);
            c1 = mfma32(qa[1][t], b, c1);
            b = bn;
        }
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float x0 = c0[j], x1 = c1[j];
            if (relu) {
                x0 = fmaxf(x0, 0.f);
                x1 = fmaxf(x1, 0.f);
            }
            acc = fmaf(wv[0][j], x0, acc);
            acc = fmaf(wv[1][j], x1, acc);
        }
        acc += __shfl_xor(acc, 32, 64);
        const int s = tile * kTile + m;
        if (g == 0 && q_ok && s < S_max) out[s] = (s < nv) ? acc * scale : mb;
    };

    load_tile(0, kt0);
    for (int tile = 0; tile < ntiles; tile += 2) {
        run_tile(tile, kt0, kt1);
        if (tile + 1 < ntiles) run_tile(tile + 1, kt1, kt0);
    }

    // the rest of the row: mask bound
    if (q_ok) {
        const int start = ntiles * kTile;
        if ((S_max & 3) == 0) {
            const f32x4v mv = {mb, mb, mb, mb};
            for (int s = start + 4 * lane; s < S_max; s += 256)
                __builtin_nontemporal_store(mv, reinterpret_cast<f32x4v*>(out + s));
        } else {
            for (int s = start + lane; s < S_max; s += 64) out[s] = mb;
        }
    }
}

}  // namespace

bool score_prefill_available() { return true; }

hipError_t launch_score_prefill(const void* q, const float* w, const void* k_cache, const int32_t* positions,
                                int32_t valid_len, int32_t M, int32_t rows_per_seq, int32_t H, int32_t S_max,
                                float scale, bool relu, float* scores, hipStream_t stream)
{
    const int n_seq = M / rows_per_seq;
    const int groups = n_seq * ((rows_per_seq + kQ - 1) / kQ);
    score_prefill_kernel<<<groups, kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(q), w, static_cast<const uint16_t*>(k_cache), positions, valid_len, rows_per_seq,
        H, S_max, scale, relu ? 1 : 0, scores);
    return hipGetLastError();
}

}  // namespace dsa
