// Top-k sparse multi-query attention with an attention sink for calls with
// many query tokens (prefill-shaped), gfx950.
//
// Definition (NeMo AutoModel deepseek_v4 optimized_kernels page,
// sparse_attention_torch; kwkr.cn article on DeepSeek-V4-Pro
// inference/kernel.py, sparse-attention section): every query head attends
// to the KV rows listed in its token's index list (-1 or out-of-range
// entries masked); the listed rows are gathered in blocks of 64 entries and
// folded into an online softmax (running max and sum-exp); the learnable
// sink adds exp(sink - max) to the denominator once, at the end.
//
// gfx950 design:
//   * workgroup = (query token, group of 128 heads), 4 waves, one per SIMD;
//     wave w owns 32 heads (two 16-head MFMA tiles) and every list entry.
//     Used when such workgroups alone fill the chip, so the list is never
//     split.  Every KV operand read from LDS feeds both head tiles, half the
//     LDS bytes per flop of 16-head waves; q for the 32 heads stays in VGPRs
//     for the whole list (144 registers), the 32 heads x 512 value features
//     of the output accumulator in AGPRs (256 registers).  On 8192 query
//     tokens x 2048 entries x 128 heads (576 / 512) this ran 4.95 ms against
//     5.97 ms for the 16-head-wave kernel of the decode calls.
//   * gather: a block's 64 listed KV rows are copied straight from HBM or L2
//     into LDS with 16-byte buffer loads (no registers), double-buffered so
//     block b+1 streams in while block b is computed (2 x 74 KB at Dqk 576).
//     Rows are padded to units with rowu % 16 == 10, which keeps the operand
//     read patterns free of LDS bank conflicts; masked entries load row 0
//     (finite data, weight 0).  The block's 64 list entries live in the
//     lanes of every wave (lane = entry): row offsets come from a lane
//     shuffle, the mask from a ballot.
//   * QK^T: v_mfma_f32_16x16x32_bf16, M = 16 entries, N = 16 heads, K = 32
//     dims, A = KV row slices (ds_read_b128), B = q.
//   * P.V: v_mfma_f32_32x32x16_bf16 (on this part it sustains about 1.6
//     PFLOP/s against 1.3 for the 16x16x32 shape), M = 32 value features,
//     N = 32 heads, K = 16 entries.  P^T comes from the QK accumulators of
//     the two head tiles with one v_permlane16_swap per register pair; V^T
//     comes from row-major LDS with ds_read_b64_tr_b16, which hands each lane
//     one value column across 4 consecutive rows.
//   * softmax in log2 units against a per-head reference max fixed at the
//     head's first live block (see the softmax below); the accumulator is
//     never rescaled.
//   * paged KV (a block table maps each page of a sequence's slots to a page
//     of a shared pool): a pool may exceed 4 GiB, which one buffer
//     descriptor cannot span (buffer offsets are 32-bit), so the paged copies
//     are global LDS loads with per-lane 64-bit addresses; a block's list
//     entries are fetched three blocks ahead and their table lookups issued
//     two blocks ahead, so the extra dependent load never stalls a copy.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kBlock = 64;      // index-list entries per block: one per lane
constexpr int kHalf = 32;       // a block whose upper half is masked skips it
constexpr int kWaves = 4;       // waves per workgroup, one per SIMD
constexpr int kWaveHeads = 32;  // heads per wave
constexpr int kHeads = kWaves * kWaveHeads;  // heads per workgroup
static_assert(kHeads == plan::kWideHeads, "the host-side plan counts workgroups of kHeads heads");
constexpr int kET = kBlock / 16;             // 16-entry tiles per block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMaxGrowth = 16.f;  // log2 units a block max may exceed the reference max
constexpr int kXcds = 8;
constexpr int kAheadQk = 3;  // K steps between a QK operand read and its MFMAs
constexpr int kAheadPv = 4;  // feature tiles between a V^T operand read and its MFMA
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kBufferWord3 = 0x00020000;  // buffer descriptor word 3: 32-bit data, raw (byte-addressed) access

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// acc += A . B (32 x 32 x 16) with the accumulator in AGPRs, as an asm
// statement: the compiler cannot keep a 256-register accumulator in AGPRs
// while the QK products write VGPRs, so the P.V products name the register
// class themselves.  The compiler does not see these as MFMAs, so the
// hazards around them are covered by hand: operands written by VALU need two
// wait states before the MFMA reads them (mfma_operand_fence), and results
// need 18 wait states before VALU, v_accvgpr_read or another writer touches
// them (mfma_result_fence).
__device__ __forceinline__ void mfma32_agpr(f32x16& acc, u32x4 a, u32x4 b)
{
    __asm__ volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_operand_fence() { __asm__ volatile("s_nop 1"); }
__device__ __forceinline__ void mfma_result_fence() { __asm__ volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"); }

// Wait until every vector-memory operation of this wave (including LDS DMA)
// has completed: vmcnt(0), expcnt / lgkmcnt unconstrained.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// max / sum over the 4 lane groups g (lanes n, n + 16, n + 32, n + 48)
__device__ __forceinline__ float group_max(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b2[0]), __uint_as_float(b2[1]));
}
__device__ __forceinline__ float group_sum(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b2[0]) + __uint_as_float(b2[1]);
}

// Gather of one block of 64 rows of ROWU units by NT threads: value =
// instructions of the busiest wave, full = leading iterations in range for
// every wave.  64 * ROWU is a multiple of 64, so a wave instruction is
// either wholly inside the block or wholly past it.
template <int ROWU, int NT>
struct GatherIters {
    static constexpr int total = kBlock * ROWU;
    static constexpr int value = (total + NT - 1) / NT;
    static constexpr int full = total / NT;
};

// KSTEPS: Dqk / 32; DT: 32-feature tiles of the value; ROWU: padded row
// length in 16-B units, ROWU % 16 == 10 (the smallest such length >= Dqk /
// 8).  With that stride both operand read patterns are free of LDS bank
// conflicts on gfx950: the 16-byte QK reads (16 rows x one unit) and the
// transposed 8-byte PV reads (4 rows x 32 bytes); odd strides such as 73
// conflict on both (measured with SQ_LDS_BANK_CONFLICT).
// EXACT: the shape is exactly (32 KSTEPS, 32 DT), so every loop has a fixed
// trip count; otherwise they are upper bounds and loops are predicated.
// PAGED: kv is a page pool addressed through pm (kv rows of sequence b at
// slot t: pool row page * 2^lp + t mod 2^lp).
template <int KSTEPS, int DT, int ROWU, bool EXACT, bool PAGED>
__global__ __launch_bounds__(kWaves * 64, 1) void sparse_attn_wide_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const float* __restrict__ sink,
    const int32_t* __restrict__ idx, int32_t BS, int32_t S, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t S_kv,
    int32_t K_top, float sm_scale, uint16_t* __restrict__ out, float* __restrict__ lse, PageMap pm)
{
    constexpr int kThreads = kWaves * 64;
    __shared__ __attribute__((aligned(16))) u32x4 kvbuf0[kBlock * ROWU];
    __shared__ __attribute__((aligned(16))) u32x4 kvbuf1[kBlock * ROWU];
    __shared__ int restart_pass;  // the pass some wave found void (see the softmax)

    // Workgroups are dealt to the XCDs round-robin (id % kXcds).  Each XCD
    // takes a run of consecutive tokens (all their head groups): tokens of one
    // sequence list overlapping KV rows, which then come from that XCD's L2.
    const int HG = (Hq + kHeads - 1) / kHeads;
    const int id = blockIdx.x;
    const int tok_per_xcd = (BS + kXcds - 1) / kXcds;
    const int local = id / kXcds;
    const int tok = (id % kXcds) * tok_per_xcd + local / HG;
    if (local >= tok_per_xcd * HG || tok >= BS) return;  // uniform
    const int hg = local % HG;
    const int b = tok / S;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int n16 = lane & 15;  // QK layout: head within a 16-head tile
    const int g = lane >> 4;    // QK layout: lane group (entries 4g .. 4g + 3 of a tile)
    const int g2 = lane >> 5;   // PV layout: lane half (features 8i + 4 g2 + j)
    const int head0 = hg * kHeads + wave_u * kWaveHeads;  // first head of this wave
    const bool wave_active = head0 < Hq;                 // wave-uniform
    const int ksteps = EXACT ? KSTEPS : Dqk / 32;
    const int dtiles = EXACT ? DT : (Dv + 31) / 32;
    const int dunits = EXACT ? 4 * KSTEPS : Dqk / 8;  // 16-B units per KV row
    const int rowu = EXACT ? ROWU : dunits + ((10 - dunits) & 15);  // padded: rowu % 16 == 10
    const int e0 = 0, e1 = K_top;  // the list is never split
    const int nblk = (K_top + kBlock - 1) / kBlock;
    const int32_t* __restrict__ ilist = idx + (size_t)tok * K_top;
    const uint16_t* __restrict__ kvb = PAGED ? kv : kv + (size_t)b * S_kv * Dqk;

    // q of this lane's heads (head0 + 16 ht + n16): B operands of QK^T (dims 32t + 8g .. +7)
    u32x4 qreg[2][KSTEPS];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
        const int h = head0 + 16 * ht + n16;
        const uint16_t* qh = q + ((size_t)tok * Hq + (h < Hq ? h : 0)) * Dqk + 8 * g;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t)
            qreg[ht][t] = (h < Hq && t < ksteps) ? *reinterpret_cast<const u32x4*>(qh + 32 * t) : u32x4{0, 0, 0, 0};
    }

    // Every wave keeps the 64 index-list entries of a block in its lanes
    // (lane = entry).  fetch_idx issues an unconditional in-bounds load;
    // check_idx turns the loaded value into a row or -1 once it is used.
    auto fetch_idx = [&](int blk) -> int {
        const int j = e0 + blk * kBlock + lane;
        return ilist[j < K_top ? j : K_top - 1];
    };
    auto check_idx = [&](int blk, int t) -> int {
        const int j = e0 + blk * kBlock + lane;
        return (blk < nblk && j < e1 && t >= 0 && t < S_kv) ? t : -1;
    };
    // Issue the LDS DMA of a block's rows (entry e's row in lane e of rows_idx)
    // into dst: the block's 64 x rowu units are walked flat, 64 consecutive
    // units per wave instruction.
    // The copies are buffer loads (MUBUF) into LDS over this sequence's KV
    // rows, not global_load_lds: the compiler treats a pending FLAT LDS copy
    // as an outstanding LDS access of unknown order and would then drain
    // every LDS operand read completely instead of counting them.  The
    // buffer's byte bound (S_kv * Dqk * 2, below 2 GiB) makes any stray
    // offset read zeros.
    const __amdgpu_buffer_rsrc_t kv_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)kvb, 0, PAGED ? 0 : (int)((long long)S_kv * Dqk * 2), kBufferWord3);
    auto gather = [&](int rows_idx, u32x4* dst) {
        const int total = kBlock * rowu;
        // byte offset of each entry's row, or its pool row when paged; a
        // masked entry reads row 0 (finite data, weight 0)
        const int eoff = PAGED ? max(rows_idx, 0) : max(rows_idx, 0) * (2 * Dqk);
        // copy of unit u0 + lane (a wave instruction covers 64 consecutive
        // units) from byte `col16` of the row at `roff`
        auto one = [&](const int u0, const int roff, const int col16) {
            if (PAGED)
                __builtin_amdgcn_global_load_lds(
                    (const void*)(reinterpret_cast<const char*>(kvb) + (size_t)(uint32_t)roff * (2 * Dqk) + col16),
                    (lds_void*)(dst + u0), 16, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(kv_rsrc, (lds_void*)(dst + u0), 16, roff + col16, 0, 0, 0);
        };
        if (EXACT) {
            constexpr int kIt = GatherIters<ROWU, kThreads>::value;
            constexpr int kFull = GatherIters<ROWU, kThreads>::full;
            // (row, column) of this lane's unit in each copy instruction, stepped
            // by kThreads units per instruction.  The lane index is made opaque so
            // that these are recomputed per block: hoisted out of the block loop
            // they would hold 2 x kIt registers for the whole list.
            int u = 64 * wave_u + lane;
            __asm__ volatile("" : "+v"(u));
            const int row0 = u / ROWU, col0 = u - row0 * ROWU;
            auto step = [](int& r, int& c) {
                c += kThreads % ROWU;
                r += kThreads / ROWU;
                if (c >= ROWU) {
                    c -= ROWU;
                    ++r;
                }
            };
            // every lane's row offsets for all of this wave's copy instructions,
            // as independent cross-lane reads, then the loads: no chain of
            // dependent steps in front of each load
            int roff[kIt];
            {
                int r = row0, c = col0;
#pragma unroll
                for (int i = 0; i < kIt; ++i) {
                    roff[i] = __builtin_amdgcn_ds_bpermute(4 * min(r, kBlock - 1), eoff);
                    step(r, c);
                }
            }
            int r = row0, c = col0;
#pragma unroll
            for (int i = 0; i < kIt; ++i) {
                const int col16 = 16 * min(c, 4 * KSTEPS - 1);  // pad unit: any valid address
                if (i < kFull || 64 * wave_u + kThreads * i < total) one(64 * wave_u + kThreads * i, roff[i], col16);
                step(r, c);
            }
        } else {
            for (int u0 = 64 * wave_u; u0 < total; u0 += kThreads) {
                const int u = u0 + lane;
                const int row = u / rowu;
                const int col = u - row * rowu;
                one(u0, __builtin_amdgcn_ds_bpermute(4 * row, eoff), 16 * min(col, dunits - 1));
            }
        }
    };

    // O^T[feature][head] of this wave's 32 heads, one 32 x 32 tile per 32
    // value features, in AGPRs.  PV layout: lane l holds head l % 32 and
    // features 32 dt + 8 i + 4 g2 + j in register 4 i + j.
    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
    float m_run[2], l_run[2];  // per head tile: reference max (log2 units), this lane's share of the sum
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
        m_run[ht] = -INFINITY;
        l_run[ht] = 0.f;
    }
    const float qk_scale = sm_scale * kLog2e;
    int pass = 0;  // passes over the list (more than one only if a max outgrows its reference)
    if (tid == 0) restart_pass = -1;  // read only after the first block barrier

    // Paged: the table entry of a checked slot (an unconditional in-bounds
    // load; a masked slot reads column 0) and the pool row it gives
    const int32_t* __restrict__ btab = PAGED ? pm.table + (size_t)b * pm.max_pages : nullptr;
    auto fetch_page = [&](int t) -> int { return PAGED ? btab[t >= 0 ? min(t >> pm.lp, pm.max_pages - 1) : 0] : 0; };
    auto pool_row = [&](int t, int page) -> int {
        return t < 0 ? -1
                     : (int)((min((uint32_t)page, (uint32_t)(pm.n_pages - 1)) << pm.lp) | (uint32_t)(t & ((1 << pm.lp) - 1)));
    };

    // Start of a pass over the list: indices of block 0 (checked) and block 1
    // (in flight), rows of block 0 (paged: block 1 checked with its table
    // lookup in flight, block 2 in flight).
    int cur_idx = 0, pending = 0, nxt_page = 0, nxt_raw = 0;
    auto start_pass = [&]() {
        cur_idx = check_idx(0, fetch_idx(0));
        pending = fetch_idx(nblk > 1 ? 1 : 0);
        if (PAGED) {
            const int page0 = fetch_page(cur_idx);
            wait_vmem();
            if (nblk > 0) gather(pool_row(cur_idx, page0), kvbuf0);
            pending = check_idx(1, pending);  // block 1: checked slot ...
            nxt_page = fetch_page(pending);   // ... and its table entry, in flight
            nxt_raw = fetch_idx(nblk > 2 ? 2 : 0);
        } else if (nblk > 0) {
            gather(cur_idx, kvbuf0);
        }
    };

    // S^T of the two 16-entry tiles from tile et0 (entries 16 et0 + m and
    // 16 et0 + 16 + m) for both head tiles.  Each A operand read feeds both
    // head tiles and is read kAheadQk K steps ahead of its MFMAs.
    auto qk_tiles = [&](const u32x4* kb, const int et0, f32x4(&s)[kET][2]) {
        constexpr int NT = 2;
#pragma unroll
        for (int c = 0; c < NT; ++c)
#pragma unroll
            for (int ht = 0; ht < 2; ++ht) s[et0 + c][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
        const u32x4* ka = kb + (16 * et0 + n16) * rowu + g;
        u32x4 ring[kAheadQk][NT];
#pragma unroll
        for (int t = 0; t < kAheadQk; ++t)
            if (t < ksteps)
#pragma unroll
                for (int c = 0; c < NT; ++c) ring[t][c] = ka[16 * c * rowu + 4 * t];
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            if (t < ksteps) {
                u32x4 x[NT];
#pragma unroll
                for (int c = 0; c < NT; ++c) x[c] = ring[t % kAheadQk][c];
                if (t + kAheadQk < ksteps)
#pragma unroll
                    for (int c = 0; c < NT; ++c) ring[t % kAheadQk][c] = ka[16 * c * rowu + 4 * (t + kAheadQk)];
#pragma unroll
                for (int c = 0; c < NT; ++c)
#pragma unroll
                    for (int ht = 0; ht < 2; ++ht) s[et0 + c][ht] = mfma16(x[c], qreg[ht][t], s[et0 + c][ht]);
            }
        }
        if (EXACT) {  // keep the reads kAheadQk K steps ahead of their MFMAs
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, NT * kAheadQk, 0);
#pragma unroll
            for (int t = 0; t < KSTEPS - kAheadQk; ++t) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * NT, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, NT, 0);
            }
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * NT * kAheadQk, 0);
        }
    };

    // O^T += V^T . P^T over the 16 entries of tile et: pb is P^T of those
    // entries (natural order, PV layout).  Transposed reads: lane group G =
    // lane / 16 covers features 32 dt + 16 (G % 2) .. +15 of rows 16 et + 8
    // (G / 2) + 0..3 and + 4..7; lane i of the group addresses row + i / 4,
    // features + 4 (i % 4) .. +3, and receives feature + i of the 4 rows.
    const int i16 = lane & 15;
    auto pv_tile = [&](const u32x4* kb, const int et, const u32x4 pb) {
        const char* vb = reinterpret_cast<const char*>(kb) +
                         (size_t)(16 * et + 8 * (g >> 1) + (i16 >> 2)) * rowu * 16 + 32 * (g & 1) + 8 * (i16 & 3);
        auto vt_operand = [&](int dt) -> u32x4 {
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + 64 * dt));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + 4 * rowu * 16 + 64 * dt));
            u32x4 a;
            a[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
            a[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
            a[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
            a[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
            return a;
        };
        u32x4 vring[kAheadPv];
#pragma unroll
        for (int dt = 0; dt < kAheadPv; ++dt)
            if (dt < dtiles) vring[dt] = vt_operand(dt);
        mfma_operand_fence();  // pb was just written by VALU
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            if (dt < dtiles) {
                const u32x4 va = vring[dt % kAheadPv];
                if (dt + kAheadPv < dtiles) vring[dt % kAheadPv] = vt_operand(dt + kAheadPv);
                mfma32_agpr(acc[dt], va, pb);
            }
        }
    };

    // One block: its rows are in kb (a compile-time choice of kvbuf0 / kvbuf1,
    // so the compiler can tell the DMA into the other buffer never aliases
    // the reads here); block blk + 1 is DMA'd into nb meanwhile.  Returns
    // whether the pass must start over (workgroup-uniform).
    auto run_block = [&](const int blk, const u32x4* kb, u32x4* nb) -> bool {
        wait_vmem();      // this wave's DMA of block blk and its index prefetch have landed
        __syncthreads();  // block blk resident for all; everyone finished block blk - 1
        if (restart_pass == pass) return true;  // a max outgrew its reference in block blk - 1
        int nxt_idx;
        if (PAGED) {
            // pending: block blk + 1's checked slots, nxt_page: their table entries,
            // nxt_raw: block blk + 2's raw entries (all landed)
            nxt_idx = pending;
            if (blk + 1 < nblk) gather(pool_row(nxt_idx, nxt_page), nb);
            pending = check_idx(blk + 2, nxt_raw);
            nxt_page = fetch_page(pending);
            nxt_raw = fetch_idx(blk + 3 < nblk ? blk + 3 : blk);
        } else {
            nxt_idx = check_idx(blk + 1, pending);
            if (blk + 1 < nblk) gather(nxt_idx, nb);
            // consumed only after the next wait_vmem, so its latency hides behind this block
            pending = fetch_idx(blk + 2 < nblk ? blk + 2 : blk);
        }
        // bit e of `valid` = entry e of the block is live
        const uint64_t valid = __ballot(cur_idx >= 0);
        cur_idx = nxt_idx;
        if (!wave_active || valid == 0) return false;  // wave-uniform: nothing to add
        const bool upper = (valid >> kHalf) != 0;  // any live entry among entries 32 .. 63

        // ---- S = KV . q^T; lane (head 16 ht + n16, group g) holds entries 16 et + 4 g + j
        f32x4 sa[kET][2];
        qk_tiles(kb, 0, sa);
        if (upper) qk_tiles(kb, 2, sa);

        // ---- online softmax per head tile, in log2 units against the
        // reference max m_run
        const uint64_t bits = valid >> (4 * g);  // entry 16 et + 4 g + j at bit 16 et + j
        uint32_t pk[kET][2][2];                  // P packed to bf16: [tile][head tile][entry pair]
        bool grow = false;
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
            float sv[kET][4];
#pragma unroll
            for (int et = 0; et < kET; ++et)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bool live = (et < 2 || upper) && ((bits >> (16 * et + j)) & 1u);
                    sv[et][j] = live ? sa[et][ht][j] * qk_scale : -INFINITY;
                }
            float bmax = -INFINITY;
#pragma unroll
            for (int et = 0; et < kET; ++et)
#pragma unroll
                for (int j = 0; j < 4; ++j) bmax = fmaxf(bmax, sv[et][j]);
            bmax = group_max(bmax);
            // Reference max: a head's first live block sets it (its accumulator is
            // still zero, so nothing needs rescaling); later blocks are weighted
            // 2^(s - m_ref) <= 2^kMaxGrowth, exact in fp32 and bf16.  A block max
            // above m_ref + kMaxGrowth asks the workgroup to run the list again
            // with the raised reference (the accumulator is never rescaled, which
            // keeps it out of VALU registers).
            if (bmax > m_run[ht] + kMaxGrowth) {
                if (m_run[ht] != -INFINITY) grow = true;
                m_run[ht] = bmax;
            }
            // The hardware exp2 (v_exp_f32, about 1 ulp) is exact enough here: its
            // argument is at most kMaxGrowth, and results below the fp32 normal
            // range only come from entries that weigh less than 2^-126 of the
            // reference.
            const float msub = (m_run[ht] == -INFINITY) ? 0.f : m_run[ht];
            float psum = 0.f;
#pragma unroll
            for (int et = 0; et < kET; ++et) {
                float p[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    p[j] = __builtin_amdgcn_exp2f(sv[et][j] - msub);
                    psum += p[j];
                }
                pk[et][ht][0] = pack_bf16x2(p[0], p[1]);
                pk[et][ht][1] = pack_bf16x2(p[2], p[3]);
            }
            l_run[ht] += psum;
        }

        if (__any(grow)) {  // this pass is void: flag it for every wave and skip P.V
            if (lane == 0) restart_pass = pass;
            return false;
        }

        // ---- O^T += V^T . P^T, one K step per 16-entry tile.  P^T in the PV
        // layout: lane l' needs head l' % 32 over entries 8 g2 .. 8 g2 + 7 of the
        // tile; the QK layout has head n16 (tile 0) and 16 + n16 (tile 1) over
        // entries 4 g .. 4 g + 3.  One permlane16 swap of the two head tiles per
        // register pair puts entries 8 g2 + 0..3 in the first and 8 g2 + 4..7 in
        // the second result.
#pragma unroll
        for (int et = 0; et < kET; ++et) {
            if (et < 2 || upper) {
                const auto s0 = __builtin_amdgcn_permlane16_swap(pk[et][0][0], pk[et][1][0], false, false);
                const auto s1 = __builtin_amdgcn_permlane16_swap(pk[et][0][1], pk[et][1][1], false, false);
                pv_tile(kb, et, u32x4{s0[0], s1[0], s0[1], s1[1]});
            }
        }
        return false;
    };
    // Scalar loads of the output pointers must not stay in flight across the
    // block loop: a pending scalar load forces every LDS wait in the loop to
    // drain completely (scalar loads may return out of order).
    __asm__ volatile("" ::"s"(out), "s"(lse), "s"(sink));
    start_pass();
    for (;;) {
        bool again = false;
        for (int blk = 0; blk < nblk && !again; blk += 2) {
            again = run_block(blk, kvbuf0, kvbuf1);
            if (!again && blk + 1 < nblk) again = run_block(blk + 1, kvbuf1, kvbuf0);
        }
        if (!again) {  // the last block may have asked for another pass too
            wait_vmem();
            __syncthreads();
            again = restart_pass == pass;
        }
        if (!again) break;
        // every DMA has landed and every wave has left the list: start over
        mfma_result_fence();  // P.V products may still be writing the accumulator
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) l_run[ht] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
        ++pass;
        start_pass();
    }
    mfma_result_fence();

    // ---- epilogue.  Per-head statistics move from the QK layout (head
    // 16 ht + n16 in every lane group) to the PV layout (head l % 32): lane l
    // takes head tile (l / 16) % 2 of its own n16.
    // The sums run over the 4 lane groups of each head tile, with every lane
    // still active.
    const float l_tot0 = group_sum(l_run[0]);
    const float l_tot1 = group_sum(l_run[1]);
    const int hsel = (lane >> 4) & 1;
    const int head = head0 + (lane & 31);
    if (head >= Hq) return;
    const float l_tot = hsel ? l_tot1 : l_tot0;
    const float m_mine = hsel ? m_run[1] : m_run[0];
    const float sk = sink ? sink[head] * kLog2e : -INFINITY;
    float den = 0.f;
    if (m_mine != -INFINITY) den = l_tot + exp2f(sk - m_mine);
    const float inv = den > 0.f ? 1.f / den : 0.f;
    uint16_t* orow = out + ((size_t)tok * Hq + head) * Dv;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        if (dt < dtiles) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int f = 32 * dt + 8 * i + 4 * g2;
                if (f < Dv) {
                    uint2 w;
                    w.x = pack_bf16x2(acc[dt][4 * i + 0] * inv, acc[dt][4 * i + 1] * inv);
                    w.y = pack_bf16x2(acc[dt][4 * i + 2] * inv, acc[dt][4 * i + 3] * inv);
                    *reinterpret_cast<uint2*>(orow + f) = w;
                }
            }
            // one tile's AGPRs at a time through VGPRs
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if (lse && g2 == 0) {
        float val;
        if (m_mine == -INFINITY) val = sink ? sink[head] : -INFINITY;
        else val = (m_mine + log2f(den)) / kLog2e;
        lse[(size_t)tok * Hq + head] = val;
    }
}

template <int KSTEPS, int DT, int ROWU, bool EXACT, bool PAGED>
hipError_t launch_variant(const void* q, const void* kv, const float* attn_sink, const int32_t* idx, int32_t B,
                          int32_t S, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t S_kv, int32_t K_top, float sm_scale,
                          void* out, float* lse, const PageMap& pm, hipStream_t stream)
{
    const int BS = B * S;
    const int HG = (Hq + kHeads - 1) / kHeads;
    const long long tok_per_xcd = (BS + kXcds - 1) / kXcds;
    const long long grid = tok_per_xcd * HG * kXcds;
    sparse_attn_wide_kernel<KSTEPS, DT, ROWU, EXACT, PAGED><<<(unsigned)grid, kWaves * 64, 0, stream>>>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv), attn_sink, idx, BS, S, Hq, Dqk, Dv, S_kv,
        K_top, sm_scale, static_cast<uint16_t*>(out), lse, pm);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_attn_wide(const void* q, const void* kv, const float* attn_sink, const int32_t* idx,
                                   int32_t B, int32_t S, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t S_kv,
                                   int32_t K_top, float sm_scale, void* out, float* lse, const PageMap* paging,
                                   hipStream_t stream)
{
    // Exact instances for the MLA shape (576 / 512) and the 192 / 128 shape;
    // any other shape (Dqk <= 576, Dv <= 512) runs a predicated instance.
    // ROWU covers Dqk / 8 + ((10 - Dqk / 8) & 15) for every Dqk an instance
    // accepts.
    const PageMap pm = paging ? *paging : PageMap{nullptr, 0, 0, 0};
#define DSA_ATTN_VARIANT(KS, DT_, RU, EX)                                                                          \
    return paging ? launch_variant<KS, DT_, RU, EX, true>(q, kv, attn_sink, idx, B, S, Hq, Dqk, Dv, S_kv, K_top,    \
                                                          sm_scale, out, lse, pm, stream)                           \
                  : launch_variant<KS, DT_, RU, EX, false>(q, kv, attn_sink, idx, B, S, Hq, Dqk, Dv, S_kv, K_top,   \
                                                           sm_scale, out, lse, pm, stream)
    if (Dqk == 576 && Dv == 512) DSA_ATTN_VARIANT(18, 16, 74, true);
    if (Dqk == 192 && Dv == 128) DSA_ATTN_VARIANT(6, 4, 26, true);
    DSA_ATTN_VARIANT(18, 16, 74, false);
#undef DSA_ATTN_VARIANT
}

}  // namespace dsa
