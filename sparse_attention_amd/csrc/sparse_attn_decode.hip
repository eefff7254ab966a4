// Top-k sparse multi-query attention with an attention sink for calls with
// few query tokens (decode), gfx950.
//
// Definition (NeMo AutoModel deepseek_v4 optimized_kernels page,
// sparse_attention_torch; kwkr.cn article on DeepSeek-V4-Pro
// inference/kernel.py, sparse-attention section): every query head attends
// to the KV rows listed in its token's index list (-1 or out-of-range
// entries masked); the listed rows are processed in blocks with an online
// softmax (running max and sum-exp, history rescaled by exp(old max - new
// max)); the learnable sink adds exp(sink - max) to the denominator once,
// at the end.
//
// gfx950 design:
//   * workgroup = (query token, group of 64 heads, split of the index list),
//     4 waves, wave w owns 16 heads.  Few tokens (decode) would leave most
//     CUs idle with one workgroup per token and head group, so the list is
//     split in nsplit parts and a combine kernel merges the partial results
//     (row max, sum and normalised output per split, kept in the workspace);
//     with enough tokens nsplit = 1 and the main kernel writes the output.
//     The grid is XCD-aware: the head groups of a (token, split) get ids on
//     the same XCD so its KV rows come from HBM once and again from L2.
//   * blocks of 32 list entries.  The pages' kernel works in 64-entry blocks;
//     on the full decode step (64 tokens, 128 heads, 1152 entries) every
//     64-entry variant measured slower here: 32-head waves with 64-entry
//     blocks ran 43.4 us + 7.9 us of combine against 37.2 us + 6.6 us for this
//     kernel.  The 64-entry kernel serves calls with many query tokens
//     (sparse_attn_wide.hip).
//   * gather: the 32 listed KV rows of a block are copied straight from HBM
//     into LDS with 16-byte buffer loads (no registers), double-buffered so
//     block b+1 streams in while block b is computed.  The copy walks the
//     block's 16-byte units flat (a wave's 64 lanes may span two rows); rows
//     are padded to 74 units (576 dims) so both MFMA operand read patterns
//     are bank-conflict free; masked entries load row 0 (finite data,
//     weight 0).
//   * QK^T: v_mfma_f32_16x16x32_bf16 with M = 16 entries, N = 16 heads,
//     K = 32 dims; A = KV row slices (ds_read_b128), B = q held in registers.
//   * P.V: the S accumulator layout (lane = head, 4 consecutive entries per
//     lane group) is the B operand P^T of the 32-entry K step directly; the
//     A operand V^T comes from row-major LDS with ds_read_b64_tr_b16, which
//     hands each lane one value column across 4 consecutive rows.
//   * softmax state in log2 units (exp2), fp32; O^T[v][head] in registers;
//     cross-lane maxima and sums use v_permlane16/32_swap (no LDS traffic).
//   * the block's 32 list entries live in the lanes of every wave (lane % 32
//     = entry): DMA row addresses come from a lane shuffle, the mask from a
//     ballot.
//   * split partial outputs are stored as bf16 and rounded once more in the
//     combine.  Measured on two tokens of the full decode step (with the
//     64-entry kernel, both ways): fp32 partials gave a worst output error
//     of 3.2e-4 and a relative L2 error of 2.4e-3, bf16 partials 3.6e-4 and
//     2.9e-3, against a tolerance of 2e-2 absolute; bf16 halves the partial
//     bytes.  For the MLA shape the partials leave through LDS (the freed KV
//     buffers): each wave transposes its 16 heads x 512 values into rows and
//     writes 16 contiguous 1 KiB rows with 16-byte stores, instead of 32
//     8-byte stores that each touch 16 rows.
//   * paged KV (a block table maps each page of a sequence's slots to a page
//     of a shared pool): a pool may exceed 4 GiB, which one buffer
//     descriptor cannot span (buffer offsets, also of structured buffers,
//     are 32-bit), so the paged copies are global LDS loads with per-lane
//     64-bit addresses; a block's list entries are fetched three blocks
//     ahead and their table lookups issued two blocks ahead, so the extra
//     dependent load never stalls a copy.  The compiler waits for all LDS
//     reads around such copies (lgkmcnt(0)), which costs the paged instance
//     about 14% against the buffer-load copies of the contiguous one.
#include <algorithm>

#include "device_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kThreads = 256;
constexpr int kHeadsPerGroup = plan::kDecodeHeadsPerGroup;  // 4 waves x 16 heads
constexpr int kBlock = plan::kDecodeBlock;                  // index-list entries per block
constexpr int kMaxSplits = plan::kDecodeMaxSplits;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kXcds = 8;
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kQkAhead = 3;  // K steps between a QK operand read and its MFMA
constexpr int kPvAhead = 3;  // tiles between a V^T operand read and its MFMA
constexpr int kSchedDsRead = 0x100;
constexpr int kBufferWord3 = 0x00020000;  // buffer descriptor word 3: 32-bit data, raw (byte-addressed) access

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

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

// Gather of one block of 32 rows of ROWU units by 4 waves of 64 lanes:
// value = instructions of the busiest wave, full = leading iterations in
// range for every wave, units = LDS buffer size (the last instruction of a
// wave may run past the block into this padding).
template <int ROWU>
struct GatherIters {
    static constexpr int total = kBlock * ROWU;
    static constexpr int value = (total + kThreads - 1) / kThreads;
    static constexpr int full = total >= kThreads ? (total - kThreads) / kThreads + 1 : 0;
    static constexpr int units = (total + 63) / 64 * 64;
};

// KSTEPS: Dqk / 32; VT: Dv / 16; ROWU: padded row length in 16-B units,
// ROWU % 16 == 10 (the smallest such length >= Dqk / 8).  With that stride
// both operand read patterns are free of LDS bank conflicts on gfx950: the
// 16-byte QK reads (16 rows x one unit) and the transposed 8-byte PV reads
// (4 rows x 32 bytes); odd strides such as 73 conflict on both (measured
// with SQ_LDS_BANK_CONFLICT).
// EXACT: the shape is exactly (32 KSTEPS, 16 VT), so every loop has a fixed
// trip count; otherwise they are upper bounds and loops are predicated.
// With nsplit > 1 the results go to part_o / part_ml instead of out / lse.
// PAGED: kv is a page pool addressed through pm (kv rows of sequence b at
// slot t: pool row page * 2^lp + t mod 2^lp).
template <int KSTEPS, int VT, int ROWU, bool EXACT, bool PAGED>
__global__ __launch_bounds__(kThreads, 1) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const float* __restrict__ sink,
    const int32_t* __restrict__ idx, int32_t BS, int32_t S, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t S_kv,
    int32_t K_top, float sm_scale, int32_t nsplit, uint16_t* __restrict__ out, float* __restrict__ lse,
    uint16_t* __restrict__ part_o, float2* __restrict__ part_ml, PageMap pm)
{
    __shared__ __attribute__((aligned(16))) u32x4 kvbuf0[GatherIters<ROWU>::units];
    __shared__ __attribute__((aligned(16))) u32x4 kvbuf1[GatherIters<ROWU>::units];

    // Workgroups are dealt to the XCDs round-robin (id % kXcds).  Each XCD
    // takes whole tokens: all head groups and splits of a token share its
    // L2, so the token's q and the gathered KV rows come from HBM once.
    const int HG = (Hq + kHeadsPerGroup - 1) / kHeadsPerGroup;
    const int id = blockIdx.x;
    const int per_tok = HG * nsplit;
    const int tok_per_xcd = (BS + kXcds - 1) / kXcds;
    const int local = id / kXcds;
    const int tok = (id % kXcds) * tok_per_xcd + local / per_tok;
    if (local >= tok_per_xcd * per_tok || tok >= BS) return;  // uniform
    const int rem = local % per_tok;
    const int hg = rem % HG;
    const int split = rem / HG;
    const int b = tok / S;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int n = lane & 15;       // MFMA column: head within the wave
    const int g = lane >> 4;       // MFMA lane group
    const int head = hg * kHeadsPerGroup + wave * 16 + n;
    const bool head_ok = head < Hq;
    const int ksteps = EXACT ? KSTEPS : Dqk / 32;
    const int vtiles = EXACT ? VT : Dv / 16;
    const int dunits = EXACT ? 4 * KSTEPS : Dqk / 8;  // 16-B units per KV row
    const int rowu = EXACT ? ROWU : dunits + ((10 - dunits) & 15);  // padded: rowu % 16 == 10
    const int nblk_all = (K_top + kBlock - 1) / kBlock;
    const int bps = (nblk_all + nsplit - 1) / nsplit;
    const int blk0 = split * bps;
    const int nblk = max(0, min(nblk_all, blk0 + bps) - blk0);
    const int32_t* __restrict__ ilist = idx + (size_t)tok * K_top;
    const uint16_t* __restrict__ kvb = PAGED ? kv : kv + (size_t)b * S_kv * Dqk;

    // Every wave keeps the 32 index-list entries of a block in its lanes
    // (lane % 32 = entry).  fetch_idx issues an unconditional in-bounds load;
    // check_idx turns the loaded value into a row or -1 once it is used.
    const int el = lane & 31;
    auto fetch_idx = [&](int blk) -> int {
        const int j = (blk0 + blk) * kBlock + el;
        return ilist[j < K_top ? j : K_top - 1];
    };
    auto check_idx = [&](int blk, int t) -> int {
        const int j = (blk0 + blk) * kBlock + el;
        return (blk < nblk && j < K_top && t >= 0 && t < S_kv) ? t : -1;
    };
    // The first two blocks' list entries go out before q: block 0's copy then
    // waits only for its entries, and q streams in meanwhile.  (The branch,
    // always taken, puts the loads in a block of their own; within one block
    // the compiler would order them after the q loads.)
    int raw0 = -1, pending = -1;
    if (K_top > 0) {
        raw0 = fetch_idx(0);
        pending = fetch_idx(nblk > 1 ? 1 : 0);
    }

    // q of this lane's head: B operand of QK^T (dims 32t + 8g .. +7); moved to
    // AGPRs once block 0's copy is issued.  Lanes of heads past Hq load head 0
    // (their scores are never stored; heads do not mix in the MFMAs), so the
    // exact shapes load without a branch.
    u32x4 qreg[KSTEPS];
    {
        const uint16_t* qh = q + ((size_t)tok * Hq + (head_ok ? head : 0)) * Dqk + 8 * g;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t)
            qreg[t] = (EXACT || t < ksteps) ? *reinterpret_cast<const u32x4*>(qh + 32 * t) : u32x4{0, 0, 0, 0};
    }
    // Issue the LDS DMA of a block's rows (entry e's row in lane e of rows_idx)
    // into dst: the block's 32 x rowu units are walked flat, 64 consecutive
    // units per wave instruction.  Iterations that are in range for every
    // wave run without a branch; the last one is guarded per wave (its lanes
    // past the block fill the buffer's padding).  With rows of at least 64
    // units a wave instruction spans at most two rows, whose indices come
    // from readlane; otherwise each lane shuffles its row index.
    // The copies are buffer loads (MUBUF) into LDS over this sequence's KV
    // rows, not global_load_lds: the compiler treats a pending FLAT LDS copy
    // as an outstanding LDS access of unknown order and would then drain
    // every LDS operand read completely instead of counting them.  The
    // buffer's byte bound (S_kv * Dqk * 2, below 2 GiB) makes any stray
    // offset read zeros.
    // (paged copies address the pool directly, see the header)
    const __amdgpu_buffer_rsrc_t kv_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)kvb, 0, PAGED ? 0 : (int)((long long)S_kv * Dqk * 2), kBufferWord3);
    auto gather = [&](int rows_idx, u32x4* dst) {
        const int total = kBlock * rowu;
        // byte offset of each entry's row, or its pool row when paged (lane e
        // and lane e + 32 hold entry e); a masked entry or padding reads row 0
        // (finite data, weight 0)
        const int eoff = PAGED ? max(rows_idx, 0) : max(rows_idx, 0) * (2 * Dqk);
        // the row of unit u of the block; units past the last row are padding
        auto row_of = [&](const int u) { const int row = u / rowu; return row < kBlock ? row : 0; };
        auto one = [&](const int u0, const int roff) {
            const int u = u0 + lane;
            const int col = u - (u / rowu) * rowu;
            const int cs = col < dunits ? col : dunits - 1;  // pad unit: any valid address
            if (PAGED)
                __builtin_amdgcn_global_load_lds(
                    (const void*)(reinterpret_cast<const char*>(kvb) + (size_t)(uint32_t)roff * (2 * Dqk) + 16 * cs),
                    (lds_void*)(dst + u0), 16, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(kv_rsrc, (lds_void*)(dst + u0), 16, roff + 16 * cs, 0, 0, 0);
        };
        constexpr int kIt = GatherIters<ROWU>::value;
        constexpr int kFull = GatherIters<ROWU>::full;
        if (EXACT) {
            // Every lane's row offsets for all of this wave's copy instructions,
            // as independent cross-lane reads, then the loads: no chain of
            // dependent scalar and vector steps in front of each load.
            int roff[kIt];
#pragma unroll
            for (int i = 0; i < kIt; ++i)
                roff[i] = __builtin_amdgcn_ds_bpermute(4 * row_of(64 * wave_u + kThreads * i + lane), eoff);
#pragma unroll
            for (int i = 0; i < kFull; ++i) one(64 * wave_u + kThreads * i, roff[i]);
#pragma unroll
            for (int i = kFull; i < kIt; ++i)
                if (64 * wave_u + kThreads * i < total) one(64 * wave_u + kThreads * i, roff[i]);
        } else {
            for (int u0 = 64 * wave_u; u0 < total; u0 += kThreads)
                one(u0, __builtin_amdgcn_ds_bpermute(4 * row_of(u0 + lane), eoff));
        }
    };

    f32x4 acc[VT];
#pragma unroll
    for (int v = 0; v < VT; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;  // reference max (log2 units)
    float l_run = 0.f;        // this lane's share of the running sum
    const float qk_scale = sm_scale * kLog2e;

    // Paged: the table entry of a checked slot (an unconditional in-bounds
    // load; a masked slot reads column 0) and the pool row it gives
    const int32_t* __restrict__ btab = PAGED ? pm.table + (size_t)b * pm.max_pages : nullptr;
    auto fetch_page = [&](int t) -> int { return PAGED ? btab[t >= 0 ? min(t >> pm.lp, pm.max_pages - 1) : 0] : 0; };
    auto pool_row = [&](int t, int page) -> int {
        return t < 0 ? -1
                     : (int)((min((uint32_t)page, (uint32_t)(pm.n_pages - 1)) << pm.lp) | (uint32_t)(t & ((1 << pm.lp) - 1)));
    };

    // prologue: indices of block 0 (checked) and block 1 (in flight), rows of block 0
    // (paged: block 1 checked with its table lookup in flight, block 2 in flight)
    int cur_idx = check_idx(0, raw0);
    int nxt_page = 0;
    if (PAGED) {
        const int page0 = fetch_page(cur_idx);
        wait_vmem();
        if (nblk > 0) gather(pool_row(cur_idx, page0), kvbuf0);
        pending = check_idx(1, pending);  // block 1: checked slot ...
        nxt_page = fetch_page(pending);   // ... and its table entry, in flight
        // the raw entries of block 2 travel in nxt_raw
    } else {
        gather(cur_idx, kvbuf0);  // unconditional (an empty split copies row 0), so raw0's load stays first
    }
    int nxt_raw = PAGED ? fetch_idx(nblk > 2 ? 2 : 0) : 0;
    // q only ever feeds MFMAs, which read AGPRs: keeping it there leaves the
    // VGPRs to the accumulator and to operand reads in flight.  (This waits for
    // the q loads, which were issued before block 0's copy.)
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) __asm__("" : "+a"(qreg[t]));

    // One block: its rows are in kb (a compile-time choice of kvbuf0 / kvbuf1,
    // so the compiler can tell the DMA into the other buffer never aliases
    // the reads here); block blk + 1 is DMA'd into nb meanwhile.
    auto run_block = [&](const int blk, const u32x4* kb, u32x4* nb) {
        wait_vmem();      // this wave's DMA of block blk and its index prefetch have landed
        __syncthreads();  // block blk resident for all; everyone finished block blk - 1
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
        const uint64_t valid = __ballot(cur_idx >= 0);
        cur_idx = nxt_idx;

        // ---- S = KV . q^T : tiles c = 0, 1 (entries 16 c + m); A operands read three K steps ahead
        f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        const u32x4* ka0 = kb + n * rowu + g;
        const u32x4* ka1 = ka0 + 16 * rowu;
        u32x4 qa0[kQkAhead], qa1[kQkAhead];
#pragma unroll
        for (int t = 0; t < kQkAhead; ++t)
            if (t < ksteps) {
                qa0[t] = ka0[4 * t];
                qa1[t] = ka1[4 * t];
            }
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            if (t < ksteps) {
                const u32x4 x0 = qa0[t % kQkAhead], x1 = qa1[t % kQkAhead];
                if (t + kQkAhead < ksteps) {
                    qa0[t % kQkAhead] = ka0[4 * (t + kQkAhead)];
                    qa1[t % kQkAhead] = ka1[4 * (t + kQkAhead)];
                }
                sacc[0] = mfma16(x0, qreg[t], sacc[0]);
                sacc[1] = mfma16(x1, qreg[t], sacc[1]);
            }
        }
        if (EXACT) {  // keep the reads three K steps ahead of their MFMAs
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kQkAhead, 0);
#pragma unroll
            for (int t = 0; t < KSTEPS - kQkAhead; ++t) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * kQkAhead, 0);
        }

        // ---- online softmax; lane (head n, group g) holds entries 16 c + 4 g + j.
        // The reference max m_run only moves when a block exceeds it by more than
        // 8 (log2 units): p = 2^(s - m_run) then stays below 256, the result is
        // unchanged, and the accumulator rescale is skipped for the whole wave.
        float sv[2][4];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) sv[c][j] = sacc[c][j] * qk_scale;
        if (valid != ~0ull) {  // masked entries (list padding, -1, out of range): logit -inf
            const uint32_t bits = (uint32_t)(valid >> (4 * g));  // entry 16 c + 4 g + j at bit 16 c + j
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (!((bits >> (16 * c + j)) & 1u)) sv[c][j] = -INFINITY;
        }
        float bmax = -INFINITY;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) bmax = fmaxf(bmax, sv[c][j]);
        bmax = group_max(bmax);
        const bool upd = bmax > m_run + 8.f;  // also true for the first finite block max
        if (__any(upd)) {
            // a real branch: without the asm statement the compiler if-converts
            // this rarely taken rescale and runs it on every block
            __asm__ volatile("" ::: "memory");
            const float m_new = upd ? bmax : m_run;
            const float alpha = upd ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;  // 0 when m_run = -inf
            l_run *= alpha;
#pragma unroll
            for (int v = 0; v < VT; ++v) acc[v] *= alpha;
            m_run = m_new;
        }
        // The hardware exp2 (v_exp_f32, about 1 ulp) is exact enough here: its
        // argument is at most 8, and results below the fp32 normal range only
        // come from entries that weigh less than 2^-126 of the block maximum.
        const float msub = (m_run == -INFINITY) ? 0.f : m_run;
        float p[2][4];
        float psum = 0.f;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                p[c][j] = __builtin_amdgcn_exp2f(sv[c][j] - msub);
                psum += p[c][j];
            }
        l_run += psum;
        const u32x4 pb = {pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                          pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])};

        // ---- O^T += V^T . P^T over the block's 32 entries (one K step)
        // transposed reads: lane i of group g addresses row R0 + i/4, value column v0 + 4 (i%4)
        const int i16 = lane & 15;
        const int r0 = 4 * g + (i16 >> 2);
        const char* vb0 = reinterpret_cast<const char*>(kb) + (size_t)r0 * rowu * 16 + 8 * (i16 & 3);
        const char* vb1 = vb0 + 16 * rowu * 16;
        auto vt_operand = [&](int v) -> u32x4 {
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb0 + 32 * v));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb1 + 32 * v));
            u32x4 a;
            a[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
            a[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
            a[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
            a[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
            return a;
        };
        u32x4 vring[kPvAhead];  // V^T operands read kPvAhead tiles ahead
#pragma unroll
        for (int v = 0; v < kPvAhead; ++v)
            if (v < vtiles) vring[v] = vt_operand(v);
#pragma unroll
        for (int v = 0; v < VT; ++v) {
            if (v < vtiles) {
                const u32x4 va = vring[v % kPvAhead];
                if (v + kPvAhead < vtiles) vring[v % kPvAhead] = vt_operand(v + kPvAhead);
                acc[v] = mfma16(va, pb, acc[v]);
            }
        }
        if (EXACT) {  // V^T reads three tiles ahead of their MFMAs
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kPvAhead, 0);
#pragma unroll
            for (int v = 0; v < VT - kPvAhead; ++v) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, kPvAhead, 0);
        }
    };
    // Scalar loads of the output pointers must not stay in flight across the
    // block loop: a pending scalar load forces every LDS wait in the loop to
    // drain completely (scalar loads may return out of order).
    __asm__ volatile("" ::"s"(out), "s"(lse), "s"(part_o), "s"(part_ml), "s"(sink));
    for (int blk = 0; blk < nblk; blk += 2) {
        run_block(blk, kvbuf0, kvbuf1);
        if (blk + 1 < nblk) run_block(blk + 1, kvbuf1, kvbuf0);
    }
    if (nblk == 0) wait_vmem();  // the index prefetch

    const float l_tot = group_sum(l_run);
    if (nsplit == 1) {
        if (!head_ok) return;
        const float sk = sink ? sink[head] * kLog2e : -INFINITY;
        float inv = 0.f, den = 0.f;
        if (m_run != -INFINITY) {
            den = l_tot + exp2f(sk - m_run);
            inv = 1.f / den;
        }
        uint16_t* orow = out + ((size_t)tok * Hq + head) * Dv;
#pragma unroll
        for (int v = 0; v < VT; ++v) {
            if (v < vtiles) {
                uint2 w;
                w.x = pack_bf16x2(acc[v][0] * inv, acc[v][1] * inv);
                w.y = pack_bf16x2(acc[v][2] * inv, acc[v][3] * inv);
                *reinterpret_cast<uint2*>(orow + 16 * v + 4 * g) = w;
            }
        }
        if (lse && g == 0) {
            float val;
            if (m_run == -INFINITY) val = sink ? sink[head] : -INFINITY;
            else val = (m_run + log2f(den)) / kLog2e;
            lse[(size_t)tok * Hq + head] = val;
        }
        return;
    }
    // partial result of this split: normalised output, (max, sum) in log2 units
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const size_t ph = ((size_t)tok * nsplit + split) * Hq + head;
    if (EXACT && VT == 32 && Hq % 64 == 0) {
        // Transposed through LDS (the KV buffers are free once every wave is
        // past its last block): each wave writes its 16 heads x 512 values
        // as 16 contiguous 1 KiB rows with 16-byte stores.  Rows are padded
        // to 1040 bytes, so the 8-byte writes of the 16 heads hit distinct banks.
        constexpr int kRowB = 1040;
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's operand reads are done
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        char* tb = reinterpret_cast<char*>(wave_u < 2 ? kvbuf0 : kvbuf1) + (wave_u & 1) * 16 * kRowB;
#pragma unroll
        for (int v = 0; v < VT; ++v) {
            uint2 w;
            w.x = pack_bf16x2(acc[v][0] * inv, acc[v][1] * inv);
            w.y = pack_bf16x2(acc[v][2] * inv, acc[v][3] * inv);
            *reinterpret_cast<uint2*>(tb + n * kRowB + 2 * (16 * v + 4 * g)) = w;
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        uint16_t* pbase = part_o + (((size_t)tok * nsplit + split) * Hq + hg * kHeadsPerGroup + wave_u * 16) * Dv;
#pragma unroll
        for (int h = 0; h < 16; ++h) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(tb + h * kRowB + 16 * lane);
            *reinterpret_cast<u32x4*>(pbase + (size_t)h * Dv + 8 * lane) = x;
        }
    } else {
        if (!head_ok) return;
        uint16_t* prow = part_o + ph * Dv;
#pragma unroll
        for (int v = 0; v < VT; ++v) {
            if (v < vtiles) {
                uint2 w;
                w.x = pack_bf16x2(acc[v][0] * inv, acc[v][1] * inv);
                w.y = pack_bf16x2(acc[v][2] * inv, acc[v][3] * inv);
                *reinterpret_cast<uint2*>(prow + 16 * v + 4 * g) = w;
            }
        }
    }
    if (head_ok && g == 0) part_ml[ph] = make_float2(m_run, l_tot);
}

// Merge the nsplit partial results of every (token, head): one wave per
// (token, head), each lane handles 8 consecutive output features.  Tokens
// are placed on the XCDs as in the main kernel (XCD x takes the x-th run of
// ceil(BS / kXcds) tokens), so a token's partial results are read back from
// the L2 that wrote them.
template <int NS>
__global__ __launch_bounds__(256) void sparse_attn_combine_kernel(
    const uint16_t* __restrict__ part_o, const float2* __restrict__ part_ml, const float* __restrict__ sink,
    int32_t BS, int32_t Hq, int32_t Dv, int32_t nsplit, uint16_t* __restrict__ out, float* __restrict__ lse)
{
    const int tok_per_xcd = (BS + kXcds - 1) / kXcds;
    const int lw = (int)((blockIdx.x / kXcds) * 4 + (threadIdx.x >> 6));  // wave within the XCD's tokens
    const int tok = (int)(blockIdx.x % kXcds) * tok_per_xcd + lw / Hq;
    if (lw >= tok_per_xcd * Hq || tok >= BS) return;  // uniform over the wave
    const int lane = threadIdx.x & 63;
    const int head = lw % Hq;
    // Every load in flight at once: the sink, the (max, sum) pairs and this
    // lane's first 8 output dims of every split (a split without entries
    // holds zeros and gets weight 0).  The loads are unconditional, from
    // clamped addresses (split 0 stands in for splits past nsplit, dim 0 for
    // lanes past Dv), so no branch makes the compiler wait between them.
    const int nsp = NS == kMaxSplits ? nsplit : NS;  // the two-split instance knows its count
    float2 ml[NS];
    u32x4 v0[NS];
    const int d0 = 8 * lane < Dv ? 8 * lane : 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const size_t ph = ((size_t)tok * nsp + (s < nsp ? s : 0)) * Hq + head;
        ml[s] = part_ml[ph];
        v0[s] = *reinterpret_cast<const u32x4*>(part_o + ph * Dv + d0);
    }
    const float sk = sink ? sink[head] * kLog2e : -INFINITY;  // (after the others: its branch waits)
    // weights by selects, so that both halves of every pair are needed at once
    float M = sk;
#pragma unroll
    for (int s = 0; s < NS; ++s) M = fmaxf(M, s < nsp ? ml[s].x : -INFINITY);
    float wgt[NS];
    float den = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const bool use = s < nsp && ml[s].y > 0.f;
        const float e = exp2f(use ? ml[s].x - M : 0.f);
        wgt[s] = use ? ml[s].y * e : 0.f;
        den += wgt[s];
    }
    if (M != -INFINITY) den += exp2f(sk - M);
    const float inv = den > 0.f ? 1.f / den : 0.f;
    uint16_t* orow = out + ((size_t)tok * Hq + head) * Dv;
    for (int d = 8 * lane; d < Dv; d += 512) {
        float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if (s < nsp) {
                const u32x4 v = d == 8 * lane ? v0[s] : *reinterpret_cast<const u32x4*>(
                    part_o + (((size_t)tok * nsp + s) * Hq + head) * Dv + d);
                const float f = wgt[s] * inv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o[2 * e] += f * bf16_lo(v[e]);
                    o[2 * e + 1] += f * bf16_hi(v[e]);
                }
            }
        }
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(o[2 * e], o[2 * e + 1]);
        *reinterpret_cast<u32x4*>(orow + d) = w;
    }
    if (lse && lane == 0) {
        float val;
        if (M == -INFINITY) val = -INFINITY;
        else if (den <= 0.f) val = sink ? sink[head] : -INFINITY;
        else val = (M + log2f(den)) / kLog2e;
        lse[(size_t)tok * Hq + head] = val;
    }
}

template <int KSTEPS, int VT, int ROWU, bool EXACT, bool PAGED>
hipError_t launch_variant(const void* q, const void* kv, const float* attn_sink, const int32_t* idx, int32_t B,
                          int32_t S, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t S_kv, int32_t K_top, float sm_scale,
                          void* out, float* lse, void* workspace, const PageMap& pm, hipStream_t stream)
{
    const int BS = B * S;
    const int HG = (Hq + kHeadsPerGroup - 1) / kHeadsPerGroup;
    const int ns = plan::attn_decode_splits(BS, Hq, K_top);
    uint16_t* part_o = nullptr;
    float2* part_ml = nullptr;
    if (ns > 1) {  // the workspace layout of plan::attn_partial_bytes
        part_o = static_cast<uint16_t*>(workspace);
        const size_t o_bytes = plan::attn_decode_partial_out_bytes(BS, 1, Hq, Dv, ns);
        part_ml = reinterpret_cast<float2*>(static_cast<char*>(workspace) + o_bytes);
    }
    const long long tok_per_xcd = (BS + kXcds - 1) / kXcds;
    const long long grid = tok_per_xcd * HG * ns * kXcds;
    sparse_attn_kernel<KSTEPS, VT, ROWU, EXACT, PAGED><<<(unsigned)grid, kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv), attn_sink, idx, BS, S, Hq, Dqk, Dv, S_kv,
        K_top, sm_scale, ns, static_cast<uint16_t*>(out), lse, part_o, part_ml, pm);
    if (ns > 1) {
        const long long waves_per_xcd = tok_per_xcd * Hq;
        const unsigned cgrid = (unsigned)((waves_per_xcd + 3) / 4 * kXcds);
        if (ns == 2)
            sparse_attn_combine_kernel<2><<<cgrid, 256, 0, stream>>>(part_o, part_ml, attn_sink, BS, Hq, Dv, ns,
                                                                    static_cast<uint16_t*>(out), lse);
        else
            sparse_attn_combine_kernel<kMaxSplits><<<cgrid, 256, 0, stream>>>(part_o, part_ml, attn_sink, BS, Hq, Dv,
                                                                             ns, static_cast<uint16_t*>(out), lse);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_attn_decode(const void* q, const void* kv, const float* attn_sink, const int32_t* idx,
                                     int32_t B, int32_t S, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t S_kv,
                                     int32_t K_top, float sm_scale, void* out, float* lse, void* workspace,
                                     const PageMap* paging, hipStream_t stream)
{
    // Exact instances for the MLA decode shape (576 / 512) and the 192 / 128
    // shape; any other shape (Dqk <= 576, Dv <= 512) runs the predicated
    // 576 / 512 instance.  ROWU covers Dqk / 8 + ((10 - Dqk / 8) & 15) for
    // every Dqk an instance accepts.
    const PageMap pm = paging ? *paging : PageMap{nullptr, 0, 0, 0};
#define DSA_ATTN_VARIANT(KS, VT_, RU, EX)                                                                          \
    return paging ? launch_variant<KS, VT_, RU, EX, true>(q, kv, attn_sink, idx, B, S, Hq, Dqk, Dv, S_kv, K_top,    \
                                                          sm_scale, out, lse, workspace, pm, stream)                \
                  : launch_variant<KS, VT_, RU, EX, false>(q, kv, attn_sink, idx, B, S, Hq, Dqk, Dv, S_kv, K_top,   \
                                                           sm_scale, out, lse, workspace, pm, stream)
    if (Dqk == 576 && Dv == 512) DSA_ATTN_VARIANT(18, 32, 74, true);
    if (Dqk == 192 && Dv == 128) DSA_ATTN_VARIANT(6, 8, 26, true);
    DSA_ATTN_VARIANT(18, 32, 74, false);
#undef DSA_ATTN_VARIANT
}

}  // namespace dsa
