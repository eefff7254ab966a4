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
//   * workgroup = 4 consecutive query rows of one sequence, one per wave
//     (one wave per SIMD); two workgroups share a CU, so one's prologue and
//     tail overlap the other's MFMA loop; groups with the longest causal
//     range go first;
//   * v_mfma_f32_32x32x16_bf16 with M = 32 heads, N = 32 keys, K = 16 dims:
//     each wave keeps its row's q (64 heads x 128 dims) in registers as the
//     A operand for the whole key loop (2 head tiles x 8 K steps); the row is
//     first copied to LDS with coalesced 16-byte DMA (loading the A layout
//     straight from memory fetches every line 8 times);
//   * the B operand comes from 128-key stages of K (32 KiB) copied HBM/L2 ->
//     LDS with 16-byte buffer loads into two distinct, double-buffered arrays,
//     one barrier per stage; 16-byte units are XOR-swizzled by key so operand
//     reads are free of bank conflicts;
//   * epilogue in registers: each lane holds 16 heads of one key per head
//     tile (accumulator row = 8 (j / 4) + 4 (lane / 32) + j % 4, column =
//     lane % 32); it applies phi, weights by w[r, h] * scale (held in
//     registers), sums, and adds the other lane half with v_permlane32_swap;
//   * software-pipelined: the MFMAs of 32-key sub-tile i overlap the epilogue
//     of sub-tile i - 1; finished scores are stored after the next stage's
//     barrier, behind that stage's key copy: loads and stores share one
//     in-order counter per wave, so each stage waits for its copy with a
//     count that leaves the score stores in flight (two buffer stores, with
//     out-of-range keys dropped by the buffer bound, so the count is fixed).
//     The copies go to an opaque LDS address and the barrier is s_barrier
//     behind that counted wait: with the compiler's own tracking, or with
//     __syncthreads (a workgroup release fence), every stage waited for all
//     of its stores (473 against 465 us at 8192 x 8192, scores bit-equal);
//   * stages past a group's causal limit are skipped; the mask-bound rest of
//     each row goes out with 16-byte stores spread over the stages.
// This per-head form serves phi = ReLU, which does not commute with the head
// sum.  With the identity activation the heads fold into one query per row
// (score_prefill_fold.hip), which needs 1/H of these flops.
#include "device_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kQ = 4;                    // query rows (waves) per workgroup; two workgroups per CU
constexpr int kThreads = 64 * kQ;
constexpr int kSub = 32;                 // keys per MFMA sub-tile
constexpr int kSubs = 4;                 // sub-tiles per stage
constexpr int kStage = kSub * kSubs;     // keys per stage (one barrier each)
constexpr int kStageU = kStage * 16;     // 16-byte units per stage
constexpr int kLoads = kStageU / kThreads;
constexpr int kBufferWord3 = 0x00020000;  // buffer descriptor word 3: 32-bit data, raw (byte-addressed) access
constexpr int kRowQU = 64 * 16;         // 16-byte units of one query row (64 heads x 128 dims)
static_assert(kLoads * kThreads == kStageU, "stage must split evenly over the workgroup");

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <bool RELU>
__global__ __launch_bounds__(kThreads, 2) void score_prefill_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ k,
    const int32_t* __restrict__ positions, int32_t valid_len, int32_t rows_per_seq, int32_t H, int32_t S_max,
    float scale, float* __restrict__ scores)
{
    // Key stage layout in LDS: key kk of the stage occupies units [16 kk, 16 kk + 16);
    // its 16-byte unit c sits at slot c ^ (kk & 15), so the 16 keys that one
    // MFMA operand read touches fall into distinct banks.  Before the key loop
    // the same buffers hold the workgroup's queries in the same swizzled
    // layout (one head per 16 units, 16 KiB per row).
    __shared__ __attribute__((aligned(16))) u32x4 kt0[kStageU];
    __shared__ __attribute__((aligned(16))) u32x4 kt1[kStageU];

    const int groups_per_seq = (rows_per_seq + kQ - 1) / kQ;
    const int gid = (int)(gridDim.x - 1 - blockIdx.x);  // late (long) groups first
    const int seq = gid / groups_per_seq;
    const int grp = gid - seq * groups_per_seq;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qi = grp * kQ + wave;
    const bool q_ok = qi < rows_per_seq;  // uniform over the wave
    const size_t r0 = (size_t)seq * rows_per_seq + grp * kQ;
    const size_t r = q_ok ? r0 + wave : r0;
    const int m = lane & 31;   // accumulator column: key within the sub-tile; A row: head within the tile
    const int g = lane >> 5;   // lane half
    const char* __restrict__ kseq = reinterpret_cast<const char*>(k + (size_t)seq * S_max * 128);

    // valid lengths of the group's rows: lane i < kQ loads row i's position
    // here and the lengths are formed after the copies below have been issued
    // (branch-free, so that nothing waits on this load early)
    const bool nl_ok = lane < kQ && grp * kQ + lane < rows_per_seq;
    const int pos_raw = positions ? positions[r0 + (nl_ok ? lane : 0)] : 0;

    // LDS DMA of stage `st`: thread tid fills slot tid % 16 of key tid / 16 + 32 i
    // (i < kLoads) with global unit slot ^ (key & 15); a wave's 64 lanes land
    // on 64 consecutive slots.
    const int dk = tid >> 4;
    const int dch = (tid & 15) ^ (dk & 15);
    const uint32_t doff = (uint32_t)(dk * 256 + 16 * dch);  // bytes within the stage
    // The copies are buffer loads (MUBUF) into LDS rather than
    // global_load_lds: with a FLAT copy in flight the compiler drains every
    // LDS operand read completely instead of counting them.  The buffer's
    // byte bound (S_max * 256, below 2 GiB) returns zeros for keys past the
    // cache, which are masked anyway.
    const __amdgpu_buffer_rsrc_t k_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)kseq, 0, S_max * 256, kBufferWord3);
    auto load_stage = [&](const int st, u32x4* dst) {
        const uint32_t base = (uint32_t)(st * kStage) * 256u + doff;
        const uint32_t d0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)(dst + 64 * wave));
#pragma unroll
        for (int i = 0; i < kLoads; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(k_rsrc, (lds_void*)(uintptr_t)(d0 + 16u * (uint32_t)(i * kThreads)),
                                                     16, base + i * (kThreads / 16) * 256, 0, 0, 0);
    };
    // The wave's query row is staged through the key buffers (rows 0-1 in kt0,
    // rows 2-3 in kt1) before the key loop.  The copy is coalesced (each
    // instruction reads 4 heads = 1 KiB); loading the A operand straight from
    // memory would fetch every 128-byte line 8 times.
    u32x4* const qs = (wave < 2 ? kt0 : kt1) + (wave & 1) * kRowQU;
    {
        const int hl = lane >> 4;                  // head within the instruction's 4
        const int cs = lane & 15;                  // slot within the head
        // heads past H read zeros (buffer bound: one row, H * 256 bytes)
        const __amdgpu_buffer_rsrc_t q_rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void*)(q + r * H * 128), 0, H * 256, kBufferWord3);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int h = 4 * i + hl;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(q_rsrc, (lds_void*)(qs + 64 * i), 16,
                                                     (uint32_t)(h * 256 + 16 * (cs ^ (h & 15))), 0, 0, 0);
        }
    }

    // the weights of the heads this lane accumulates (32 mt + 8 jj + 4 g + i),
    // pre-multiplied by scale
    float wv[2][16];
    // (unconditional loads from clamped addresses, zeroed by selects: no
    // divergent branch forces an early wait)
    const float* wr = w + r * H;
    if ((H & 3) == 0) {  // uniform: 16-byte loads
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int h0 = 32 * mt + 8 * jj + 4 * g;
                const float4 v4 = *reinterpret_cast<const float4*>(wr + (h0 < H ? h0 : 0));
                const float f = (q_ok && h0 < H) ? scale : 0.f;
                wv[mt][4 * jj + 0] = v4.x * f;
                wv[mt][4 * jj + 1] = v4.y * f;
                wv[mt][4 * jj + 2] = v4.z * f;
                wv[mt][4 * jj + 3] = v4.w * f;
            }
    } else {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int hh = 32 * mt + 8 * (i >> 2) + 4 * g + (i & 3);
                const float v = wr[hh < H ? hh : 0];
                wv[mt][i] = v * ((q_ok && hh < H) ? scale : 0.f);
            }
    }

    int nl = S_max;
    if (positions) nl = pos_raw < S_max ? pos_raw + 1 : S_max;  // no overflow: pos_raw + 1 <= S_max
    if (valid_len >= 0 && valid_len < nl) nl = valid_len;
    nl = nl_ok ? max(nl, 0) : 0;
    int nv = 0, nv_max = 0;
#pragma unroll
    for (int i = 0; i < kQ; ++i) {
        const int n = __builtin_amdgcn_readlane(nl, i);
        nv_max = max(nv_max, n);
        if (i == wave) nv = n;
    }
    const int nstages = (nv_max + kStage - 1) / kStage;

    // A operand from the staged row: q[r][32 mt + m][16 t + 8 g .. +7]
    wait_vmem();
    u32x4 qa[2][8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const int h = 32 * mt + m;
        const bool h_ok = q_ok && h < H;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const u32x4 v = qs[h * 16 + ((g + 2 * t) ^ (h & 15))];
            qa[mt][t] = h_ok ? v : u32x4{0, 0, 0, 0};
        }
    }

    __syncthreads();  // every wave has its A operand: the key buffers are free
    load_stage(0, kt0);

    // operand read offsets: lane (m, g) reads unit g + 2 t of key m
    int rd[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) rd[t] = m * 16 + ((g + 2 * t) ^ (m & 15));

    const float mb = mask_bound();
    float* __restrict__ out = scores + r * S_max;
    // The mask-bound tail of the row, [nstages * kStage, S_max), goes out in
    // one chunk per stage (16-byte stores) so that it overlaps the MFMA work.
    const bool vec_rows = q_ok && (S_max & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
    const int tail0 = min(nstages * kStage, S_max);
    const int chunk = (vec_rows && nstages > 0) ? ((S_max - tail0 + nstages - 1) / nstages + 255) & ~255 : 0;

    // Software pipeline over sub-tiles: the MFMAs of sub-tile i go to one
    // accumulator pair while the epilogue of sub-tile i - 1 reduces the other.
    // Finished scores wait in sc[i % 4] and are stored after the next stage's
    // barrier, so the wait for a stage's DMA never waits on recent stores.
    f32x16 acc[2][2];
#pragma unroll
    for (int p = 0; p < 2; ++p) acc[p][0] = acc[p][1] = f32x16{};
    float sc[4] = {0.f, 0.f, 0.f, 0.f};

    auto mfma_sub = [&](const u32x4* kb, f32x16& c0, f32x16& c1) {
        c0 = f32x16{};
        c1 = f32x16{};
        u32x4 b = kb[rd[0]];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const u32x4 bn = (t + 1 < 8) ? kb[rd[(t + 1) & 7]] : b;
            c0 = mfma32(qa[0][t], b, c0);
            c1 = mfma32(qa[1][t], b, c1);
            b = bn;
        }
    };
    auto epilogue = [&](const f32x16& c0, const f32x16& c1) {
        // four independent partial sums
        float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float x0 = c0[j], x1 = c1[j];
            if (RELU) {
                x0 = fmaxf(x0, 0.f);
                x1 = fmaxf(x1, 0.f);
            }
            p[2 * (j & 1)] = fmaf(wv[0][j], x0, p[2 * (j & 1)]);
            p[2 * (j & 1) + 1] = fmaf(wv[1][j], x1, p[2 * (j & 1) + 1]);
        }
        const float a = (p[0] + p[1]) + (p[2] + p[3]);
        // add the other lane half: v_permlane32_swap exchanges the halves of two copies
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
        return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    };
    // At the start of stage st the scores of sub-tiles 4 st - 5 .. 4 st - 2 are
    // final (slot 3 holds 4 st - 5, slot j < 3 holds 4 st - 4 + j); they go
    // out as two runs of 64 keys: (4 st - 5, 4 st - 4) and (4 st - 3, 4 st - 2).
    const __amdgpu_buffer_rsrc_t o_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)out, 0, q_ok ? S_max * 4 : 0, kBufferWord3);
    auto flush = [&](const int st) {
        const int k0 = kSub * (kSubs * st - 5);
        const float va = g ? sc[0] : sc[3];
        const float vb = g ? sc[2] : sc[1];
        const int sa = k0 + lane, sb = k0 + 2 * kSub + lane;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sa < nv ? va : mb), o_rsrc,
                                              (sa >= 0 && sa < S_max) ? (uint32_t)sa * 4u : 0x80000000u, 0, 2);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sb < nv ? vb : mb), o_rsrc,
                                              (sb >= 0 && sb < S_max) ? (uint32_t)sb * 4u : 0x80000000u, 0, 2);
    };
    auto stage = [&](const int st, const u32x4* cur, u32x4* nxt) {
        // This wave's copy of stage st has landed: after it only the two score
        // stores of the previous stage were issued (stage 0: nothing), so the
        // count leaves them in flight.  A __syncthreads (a workgroup release
        // fence) would wait for every copy and store instead.
        if (st == 0) __builtin_amdgcn_s_waitcnt(0x0070);            // vmcnt(0) lgkmcnt(0)
        else __builtin_amdgcn_s_waitcnt(2 | (7 << 4));              // vmcnt(2) lgkmcnt(0)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();  // stage resident for all waves; everyone finished reading the other buffer
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (vec_rows) {
            const f32x4v mv = {mb, mb, mb, mb};
            const int e = min(S_max, tail0 + (st + 1) * chunk);
            for (int s = tail0 + st * chunk + 4 * lane; s < e; s += 256)
                __builtin_nontemporal_store(mv, reinterpret_cast<f32x4v*>(out + s));
        }
        if (st + 1 < nstages) load_stage(st + 1, nxt);
        flush(st);
#pragma unroll
        for (int j = 0; j < kSubs; ++j) {
            mfma_sub(cur + j * kSub * 16, acc[j & 1][0], acc[j & 1][1]);
            sc[(j + 3) & 3] = epilogue(acc[(j + 1) & 1][0], acc[(j + 1) & 1][1]);
        }
    };

    for (int st = 0; st < nstages; st += 2) {
        stage(st, kt0, kt1);
        if (st + 1 < nstages) stage(st + 1, kt1, kt0);
    }
    if (nstages > 0) {
        flush(nstages);
        sc[3] = epilogue(acc[1][0], acc[1][1]);
        const int s = kSub * (kSubs * nstages - 1) + m;
        if (g == 0 && q_ok && s < S_max) out[s] = (s < nv) ? sc[3] : mb;
    } else {
        wait_vmem();  // the stage-0 copy must land before the workgroup's LDS is released
    }

    // the rest of the row when it did not go out with the stages
    if (q_ok && !(vec_rows && nstages > 0)) {
        if (vec_rows) {
            const f32x4v mv = {mb, mb, mb, mb};
            for (int s = tail0 + 4 * lane; s < S_max; s += 256)
                __builtin_nontemporal_store(mv, reinterpret_cast<f32x4v*>(out + s));
        } else {
            for (int s = tail0 + lane; s < S_max; s += 64) out[s] = mb;
        }
    }
}

}  // namespace


hipError_t launch_score_prefill(const void* q, const float* w, const void* k_cache, const int32_t* positions,
                                int32_t valid_len, int32_t M, int32_t rows_per_seq, int32_t H, int32_t S_max,
                                float scale, float* scores, hipStream_t stream)
{
    // the identity activation folds over heads instead (score_prefill_fold.hip)
    const int n_seq = M / rows_per_seq;
    const int groups = n_seq * ((rows_per_seq + kQ - 1) / kQ);
    auto* qp = static_cast<const uint16_t*>(q);
    auto* kp = static_cast<const uint16_t*>(k_cache);
    score_prefill_kernel<true><<<groups, kThreads, 0, stream>>>(qp, w, kp, positions, valid_len, rows_per_seq, H,
                                                                S_max, scale, scores);
    return hipGetLastError();
}

}  // namespace dsa

