// Decode lightning-indexer score with the per-head activation max(0, .), for
// gfx950 (one query row per sequence).
//
// Definition (AWS Neuron "DeepSeek-V3.2 Sparse Indexer Kernel API
// Reference", Returns and Notes): every cached key slot s < n_valid(r) of
// row r gets
//   score = scale * sum_h w[r,h] * relu(q[r,h,:] . K[r,s,:])
// and the others the finite mask bound.  max(0, .) does not commute with
// the head sum, so unlike the identity case (score_decode.hip) the heads
// cannot be folded into one query: every slot needs H dot products.
//
// That is 2 * 64 * 128 flop per 256-byte bf16 slot (64 flop/B), far below
// the MFMA ridge, so the kernel stays a stream over the key cache, with the
// per-head contraction on MFMA:
//   * grid (runs of cpw chunks of 512 slots, rows), 4 waves; in every chunk
//     wave w scores slots [128 w, 128 w + 128) as 8 tiles of 16 slots.  A
//     workgroup loads the row's q once and keeps its key loads in flight
//     across its chunks: with one chunk per workgroup the first loads'
//     latency, paid by every workgroup, held the stream near 55% of HBM
//     bandwidth, and runs sized to give about one resident wave of
//     workgroups (two per CU) reach about 72%;
//   * v_mfma_f32_16x16x32_bf16 with M = 16 heads (up to 4 head tiles),
//     N = 16 slots, K = 32 dims: the row's q is the A operand for the whole
//     chunk (16 register quads), the keys are the B operand loaded straight
//     from memory, four tiles in flight.  Every key load is issued without a
//     branch around it (lanes past the attendable slots read the tile's last
//     one, and a wave past its last tile reloads that tile), so the compiler
//     counts them and each tile waits for its own loads: with the loads under
//     per-lane and per-tile branches every tile drained all of them (4 x
//     131072 fp8 slots: 20.6 against 31.8 us; 16 x 32768 bf16: 26.7 against
//     27.5 us; scores bit-equal).  bf16 keys: lane (slot n, group g)
//     takes dims 32 t + 8 g .. + 7 in K step t (64 contiguous bytes of the
//     slot per wave load);
//   * fp8 keys: lane (n, g) loads bytes 32 g .. 32 g + 31 of the slot and
//     converts them exactly to bf16 (every E4M3 value is a bf16 value), so
//     its K step t covers dims 32 g + 8 t; q is loaded in the same order.
//     The slot's scale multiplies its dot products before the activation;
//   * epilogue in registers: lane (n, g) holds heads 16 ht + 4 g + j of
//     slot n; it applies max(0, .), weights by w[h] * scale, sums its heads,
//     and the four lane groups are added with lane swaps;
//   * scores are staged in LDS and written with 16-byte stores; chunks past
//     n_valid only write the mask bound;
//   * like the folded scorer, the launch can clear an unrelated buffer (the
//     top-k workspace header of a decode step) on the side;
//   * paged caches: a 16-slot tile never straddles a page (pages are a power
//     of two >= 64 slots), so one table lookup per tile gives its rows.
#include "device_common.h"
#include "dsa_internal.h"

#include <algorithm>

namespace dsa {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 512;         // slots per workgroup
constexpr int kMaxCpw = 16;         // chunks per workgroup at most
constexpr int kTargetWgs = 512;     // two resident workgroups on each of 256 CUs
constexpr int kAhead = 4;           // tiles in flight per wave
constexpr int kMaxHeadTiles = 4;    // H <= 64

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// sum over the 4 lane groups of an MFMA column (lanes n, n + 16, n + 32, n + 48)
__device__ __forceinline__ float lane_group_sum(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 8 E4M3 codes (two 32-bit words) -> 8 bf16 (one B operand quad), exact
__device__ __forceinline__ u32x4 fp8x8_to_bf16(uint32_t lo, uint32_t hi)
{
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
    const auto d = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
    return u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(b[0], b[1]), pack_bf16x2(c[0], c[1]),
                 pack_bf16x2(d[0], d[1])};
}

template <bool FP8, bool PAGED>
__global__ __launch_bounds__(kThreads, 2) void score_decode_heads_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint8_t* __restrict__ k,
    const float* __restrict__ k_scale, const int32_t* __restrict__ positions, int32_t valid_len, int32_t H,
    int32_t S_max, int32_t cpw, float scale, float* __restrict__ scores, uint32_t* __restrict__ zero_ptr,
    size_t zero_words, PageMap pm)
{
    clear_words(zero_ptr, zero_words);
    __shared__ __attribute__((aligned(16))) float stage[kChunk * kMaxCpw];
    const int r = blockIdx.y;
    const int s0 = blockIdx.x * kChunk * cpw;
    const int s1 = min(s0 + kChunk * cpw, S_max);
    const int n_tiles = 8 * cpw;  // per wave
    const int nv = n_valid_of(positions, valid_len, r, S_max);
    float* __restrict__ out = scores + (size_t)r * S_max;

    const float mb = mask_bound();
    for (int s = max(s0, nv) + (int)threadIdx.x; s < s1; s += kThreads) out[s] = mb;
    const int se = min(s1, nv);
    if (s0 >= se) return;  // uniform over the workgroup

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;  // MFMA column (slot of a tile) / A row (head of a tile)
    const int g = lane >> 4;  // lane group
    const int nht = (H + 15) >> 4;
    constexpr int kSlotBytes = FP8 ? 128 : 256;

    // The wave's tiles that hold an attendable slot: tiles 0 .. n_my - 1
    // (tile bases grow with the tile index).
    const int wbase = s0 + 128 * wave;
    auto tile_base = [&](const int i) { return wbase + kChunk * (i >> 3) + 16 * (i & 7); };
    int n_my = 0;
    while (n_my < n_tiles && tile_base(n_my) < se) ++n_my;

    // q as A operands: head tile ht, K step t, lane (head n, group g); dims
    // 32 t + 8 g (bf16 keys) or 32 g + 8 t (fp8 keys, see the header).  Loaded
    // first, so the first tile's wait does not reach past them.
    u32x4 qa[kMaxHeadTiles][4];
    float wsc[kMaxHeadTiles][4];  // w[16 ht + 4 g + j] * scale
    const uint16_t* __restrict__ qr = q + (size_t)r * H * 128;
    const float* __restrict__ wr = w + (size_t)r * H;
#pragma unroll
    for (int ht = 0; ht < kMaxHeadTiles; ++ht) {
        const int h = 16 * ht + n;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int d = FP8 ? 32 * g + 8 * t : 32 * t + 8 * g;
            const u32x4 x = *reinterpret_cast<const u32x4*>(qr + (size_t)(h < H ? h : 0) * 128 + d);
            qa[ht][t] = h < H ? x : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int hw = 16 * ht + 4 * g + j;
            const float wh = wr[hw < H ? hw : 0];  // unconditional: no branch, no early wait
            wsc[ht][j] = hw < H ? wh * scale : 0.f;
        }
    }

    // Keys of tile i (slots sb .. sb + 15) as four B operands (fp8: its codes,
    // converted at use, and the slot scales).  Every lane loads: slots past
    // se read the tile's last attendable slot (same tile, so the same page),
    // and their scores are never kept.  With no branch around the loads the
    // compiler counts them and each tile waits for its own loads alone.
    auto load_tile = [&](const int i, u32x4 (&kb)[4], float& ksc) {
        const int sb = tile_base(i);
        const int dn = min(sb + n, se - 1) - sb;
        const size_t row = store_row<PAGED>(pm, r, sb, S_max) + dn;
        const uint8_t* p = k + row * kSlotBytes;
        if (FP8) {
            const u32x4 x0 = *reinterpret_cast<const u32x4*>(p + 32 * g);
            const u32x4 x1 = *reinterpret_cast<const u32x4*>(p + 32 * g + 16);
            kb[0] = u32x4{x0[0], x0[1], 0u, 0u};
            kb[1] = u32x4{x0[2], x0[3], 0u, 0u};
            kb[2] = u32x4{x1[0], x1[1], 0u, 0u};
            kb[3] = u32x4{x1[2], x1[3], 0u, 0u};
            ksc = k_scale[row];
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) kb[t] = *reinterpret_cast<const u32x4*>(p + 64 * t + 16 * g);
            ksc = 1.f;
        }
    };
    u32x4 ring[kAhead][4];
    float kring[kAhead];
    if (n_my > 0) {  // uniform over the wave
#pragma unroll
        for (int u = 0; u < kAhead; ++u) load_tile(min(u, n_my - 1), ring[u], kring[u]);
#pragma unroll 1
        for (int i0 = 0; i0 < n_my; i0 += kAhead) {
#pragma unroll
            for (int u = 0; u < kAhead; ++u) {
                const int i = i0 + u;
                u32x4 kb[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) kb[t] = ring[u][t];
                const float ks = kring[u];
                // the wave's tile kAhead on (its last one again at the end): every
                // step issues the same loads
                load_tile(min(i + kAhead, n_my - 1), ring[u], kring[u]);
                if (i < n_my) {  // uniform over the wave
                    const int sb = tile_base(i);
                    if (FP8) {
#pragma unroll
                        for (int t = 0; t < 4; ++t) kb[t] = fp8x8_to_bf16(kb[t][0], kb[t][1]);
                    }
                    float acc = 0.f;
#pragma unroll
                    for (int ht = 0; ht < kMaxHeadTiles; ++ht) {
                        if (ht < nht) {  // uniform
                            f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int t = 0; t < 4; ++t) c = mfma16(qa[ht][t], kb[t], c);
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                acc = fmaf(wsc[ht][j], fmaxf(FP8 ? c[j] * ks : c[j], 0.f), acc);
                        }
                    }
                    acc = lane_group_sum(acc);
                    if (g == 0 && sb + n < se) stage[sb + n - s0] = acc;
                }
            }
        }
    }

    __syncthreads();
    if (se - s0 == kChunk * cpw && (reinterpret_cast<uintptr_t>(out + s0) & 15) == 0) {
        for (int i = threadIdx.x; i < kChunk * cpw / 4; i += kThreads)
            __builtin_nontemporal_store(reinterpret_cast<const u32x4*>(stage)[i],
                                        reinterpret_cast<u32x4*>(out + s0) + i);
    } else {
        for (int i = threadIdx.x; i < se - s0; i += kThreads) out[s0 + i] = stage[i];
    }
}

}  // namespace

hipError_t launch_score_decode_heads(const void* q, const float* w, const void* k_cache, const float* k_scale,
                                     bool key_fp8, const int32_t* positions, int32_t valid_len, int32_t M,
                                     int32_t H, int32_t S_max, float scale, float* scores, uint32_t* zero_ptr,
                                     size_t zero_words, const PageMap* paging, hipStream_t stream)
{
    const int chunks = (S_max + kChunk - 1) / kChunk;
    const long long total = (long long)chunks * M;
    const int cpw = (int)std::min<long long>(kMaxCpw, std::max<long long>(1, (total + kTargetWgs - 1) / kTargetWgs));
    const dim3 grid((chunks + cpw - 1) / cpw, M);
    const PageMap pm = paging ? *paging : PageMap{nullptr, 0, 0, 0};
    const auto* qq = static_cast<const uint16_t*>(q);
    const auto* kc = static_cast<const uint8_t*>(k_cache);
#define DSA_HEADS_LAUNCH(F8, PG)                                                                                  \
    score_decode_heads_kernel<F8, PG><<<grid, kThreads, 0, stream>>>(qq, w, kc, F8 ? k_scale : nullptr, positions, \
                                                                     valid_len, H, S_max, cpw, scale, scores,      \
                                                                     zero_ptr, zero_words, pm)
    if (key_fp8) {
        if (paging) DSA_HEADS_LAUNCH(true, true);
        else DSA_HEADS_LAUNCH(true, false);
    } else {
        if (paging) DSA_HEADS_LAUNCH(false, true);
        else DSA_HEADS_LAUNCH(false, false);
    }
#undef DSA_HEADS_LAUNCH
    return hipGetLastError();
}

}  // namespace dsa
