// Top-k sparse multi-query attention with an attention sink, gfx950.
//
// Definition (NeMo AutoModel deepseek_v4 optimized_kernels page,
// sparse_attention_torch; kwkr.cn article on DeepSeek-V4-Pro
// inference/kernel.py, sparse-attention section): every query head attends
// to the KV rows listed in its token's index list (-1 or out-of-range
// entries masked); the listed rows are processed in 64-entry blocks with an
// online softmax (running max and sum-exp, history rescaled by
// exp(old max - new max)); the learnable sink adds exp(sink - max) to the
// denominator once, at the end.
//
// gfx950 design:
//   * workgroup = (query token, group of 32 heads), 4 waves; wave w owns
//     16 heads (w & 1) and one half of every 64-entry block (w >> 1), with
//     its own online-softmax state; the two halves are merged through LDS at
//     the end, so no partial results go to HBM.  The grid is XCD-aware:
//     workgroup ids are dealt to the 8 XCDs round-robin, and all head groups
//     of a token get ids on the same XCD so its KV rows are fetched from HBM
//     once and re-read from that XCD's L2.
//   * gather: the 64 listed KV rows of a block are copied straight from HBM
//     into LDS with 16-byte global_load_lds (no registers), double-buffered
//     so block b+1 streams in while block b is computed.  Rows are padded to
//     an odd number of 16-byte units so MFMA operand reads are bank-conflict
//     free.  Masked entries load row 0 (finite data) and get weight 0.
//   * QK^T: v_mfma_f32_16x16x32_bf16 with M = 16 entries, N = 16 heads,
//     K = 32 dims; A = KV row slices (ds_read_b128), B = q held in registers.
//   * P.V: the S accumulator layout (lane = head, 4 consecutive entries per
//     lane group) is the B operand P^T of a 32-entry K step directly; the A
//     operand V^T comes from row-major LDS with ds_read_b64_tr_b16, which
//     hands each lane one value column across 4 consecutive rows.
//   * softmax state in log2 units (exp2), fp32; O^T[v][head] in registers.
//   * the block's 64 list entries live in the lanes of every wave (lane =
//     entry): DMA row addresses come from readlane, the mask from a ballot.
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
constexpr int kHeadsPerGroup = 32;
constexpr int kBlock = 64;            // index-list entries per block
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kXcds = 8;

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// Wait until every vector-memory operation of this wave (including LDS DMA)
// has completed: vmcnt(0), expcnt / lgkmcnt unconstrained.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// KSTEPS: Dqk / 32; VT: Dv / 16; ROWU: padded row length in 16-B units (odd).
// EXACT: the shape is exactly (32 KSTEPS, 16 VT), so every loop has a fixed
// trip count; otherwise they are upper bounds and loops are predicated.
template <int KSTEPS, int VT, int ROWU, bool EXACT>
__global__ __launch_bounds__(kThreads, 1) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const float* __restrict__ sink,
    const int32_t* __restrict__ idx, int32_t BS, int32_t S, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t S_kv,
    int32_t K_top, float sm_scale, uint16_t* __restrict__ out, float* __restrict__ lse)
{
    __shared__ __attribute__((aligned(16))) u32x4 kvbuf0[kBlock * ROWU];
    __shared__ __attribute__((aligned(16))) u32x4 kvbuf1[kBlock * ROWU];

    const int HG = (Hq + kHeadsPerGroup - 1) / kHeadsPerGroup;
    const int id = blockIdx.x;
    const int slot = id / kXcds;
    const int hg = slot % HG;
    const int tok = (slot / HG) * kXcds + id % kXcds;  // b * S + s
    if (tok >= BS) return;  // uniform
    const int b = tok / S;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n = lane & 15;       // MFMA column: head within the wave
    const int g = lane >> 4;       // MFMA lane group
    const int eh = wave >> 1;      // entry half of each block
    const int head = hg * kHeadsPerGroup + (wave & 1) * 16 + n;
    const bool head_ok = head < Hq;
    const int ksteps = EXACT ? KSTEPS : Dqk / 32;
    const int vtiles = EXACT ? VT : Dv / 16;
    const int dunits = EXACT ? 4 * KSTEPS : Dqk / 8;  // 16-B units per KV row
    const int rowu = EXACT ? ROWU : (dunits + 1) | 1;  // padded, odd
    const int nblk = (K_top + kBlock - 1) / kBlock;
    const int32_t* __restrict__ ilist = idx + (size_t)tok * K_top;
    const uint16_t* __restrict__ kvb = kv + (size_t)b * S_kv * Dqk;

    // q of this lane's head: B operand of QK^T (dims 32t + 8g .. +7)
    u32x4 qreg[KSTEPS];
    {
        const uint16_t* qh = q + ((size_t)tok * Hq + (head_ok ? head : 0)) * Dqk + 8 * g;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t)
            qreg[t] = (head_ok && t < ksteps) ? *reinterpret_cast<const u32x4*>(qh + 32 * t) : u32x4{0, 0, 0, 0};
    }

    // Every wave keeps the 64 index-list entries of a block in its lanes
    // (lane = entry).  fetch_idx issues an unconditional in-bounds load;
    // check_idx turns the loaded value into a row or -1 once it is used.
    auto fetch_idx = [&](int blk) -> int {
        const int j = blk * kBlock + lane;
        return ilist[j < K_top ? j : K_top - 1];
    };
    auto check_idx = [&](int blk, int t) -> int {
        const int j = blk * kBlock + lane;
        return (j < K_top && t >= 0 && t < S_kv) ? t : -1;
    };
    // Issue the LDS DMA of a block's rows (row r's index in lane r of rows_idx)
    // into dst.  Wave w copies rows 16w .. 16w + 15; per row, one instruction
    // per 64 consecutive 16-B units (the row index is wave-uniform, read with
    // readlane, so the address is a scalar base plus the lane's offset).
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    auto gather = [&](int rows_idx, u32x4* dst) {
        const char* gbase = reinterpret_cast<const char*>(kvb);
        for (int rr = 0; rr < kBlock / 4; ++rr) {
            const int row = wave_u * (kBlock / 4) + rr;
            int r = __builtin_amdgcn_readlane(rows_idx, row);
            r = r >= 0 ? r : 0;  // masked entry: row 0 (finite data, weight 0)
            const char* src = gbase + (size_t)r * (2 * Dqk);
            u32x4* d = dst + row * rowu;
            for (int c0 = 0; c0 < rowu; c0 += 64) {
                const int c = c0 + lane;
                if (c < rowu) {
                    const int cs = c < dunits ? c : dunits - 1;  // pad unit: any valid address
                    __builtin_amdgcn_global_load_lds(src + 16 * cs, (lds_void*)(d + c0), 16, 0, 0);
                }
            }
        }
    };

    f32x4 acc[VT];
#pragma unroll
    for (int v = 0; v < VT; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;  // reference max (log2 units)
    float l_run = 0.f;        // this lane's share of the running sum
    const float qk_scale = sm_scale * kLog2e;

    // prologue: indices of block 0 (checked) and block 1 (in flight), rows of block 0
    int cur_idx = check_idx(0, fetch_idx(0));
    int pending = fetch_idx(nblk > 1 ? 1 : 0);
    gather(cur_idx, kvbuf0);

    // One block: its rows are in kb (a compile-time choice of kvbuf0 / kvbuf1,
    // so the compiler can tell the DMA into the other buffer never aliases
    // the reads here); block blk + 1 is DMA'd into nb meanwhile.
    auto run_block = [&](const int blk, const u32x4* kb, u32x4* nb) {
        wait_vmem();      // this wave's DMA of block blk and its index prefetch have landed
        __syncthreads();  // block blk resident for all; everyone finished block blk - 1
        const int nxt_idx = check_idx(blk + 1, pending);
        if (blk + 1 < nblk) gather(nxt_idx, nb);
        // consumed only after the next wait_vmem, so its latency hides behind this block
        pending = fetch_idx(blk + 2 < nblk ? blk + 2 : blk);
        const uint64_t valid = __ballot(cur_idx >= 0);
        cur_idx = nxt_idx;

        // ---- S = KV . q^T : tiles c = 0, 1 (entries 32 eh + 16 c + m); operands read one K step ahead
        f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        const u32x4* ka0 = kb + (32 * eh + n) * rowu + g;
        const u32x4* ka1 = ka0 + 16 * rowu;
        u32x4 a0 = ka0[0], a1 = ka1[0];
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            if (t < ksteps) {
                u32x4 b0 = a0, b1 = a1;
                if (t + 1 < ksteps) {
                    b0 = ka0[4 * (t + 1)];
                    b1 = ka1[4 * (t + 1)];
                }
                sacc[0] = mfma16(a0, qreg[t], sacc[0]);
                sacc[1] = mfma16(a1, qreg[t], sacc[1]);
                a0 = b0;
                a1 = b1;
            }
        }

        // ---- online softmax; lane (head n, group g) holds entries 32 eh + 16 c + 4 g + j.
        // The reference max m_run only moves when a block exceeds it by more than
        // 8 (log2 units): p = 2^(s - m_run) then stays below 256, the result is
        // unchanged, and the accumulator rescale is skipped for the whole wave.
        float sv[2][4];
        float bmax = -INFINITY;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = 32 * eh + 16 * c + 4 * g + j;
                const float x = ((valid >> e) & 1) ? sacc[c][j] * qk_scale : -INFINITY;
                sv[c][j] = x;
                bmax = fmaxf(bmax, x);
            }
        bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
        bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
        const bool upd = bmax > m_run + 8.f;  // also true for the first finite block max
        if (__any(upd)) {
            // a real branch: without the asm statement the compiler if-converts
            // this rarely taken rescale and runs it on every block
            __asm__ volatile("" ::: "memory");
            const float m_new = upd ? bmax : m_run;
            const float alpha = upd ? exp2f(m_run - m_new) : 1.f;  // 0 when m_run = -inf
            l_run *= alpha;
#pragma unroll
            for (int v = 0; v < VT; ++v) acc[v] *= alpha;
            m_run = m_new;
        }
        const float msub = (m_run == -INFINITY) ? 0.f : m_run;
        float p[2][4];
        float psum = 0.f;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                p[c][j] = exp2f(sv[c][j] - msub);
                psum += p[c][j];
            }
        l_run += psum;
        const u32x4 pb = {pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                          pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])};

        // ---- O^T += V^T . P^T over this wave's 32 entries (one K step)
        // transposed reads: lane i of group g addresses row R0 + i/4, value column v0 + 4 (i%4)
        const int i16 = lane & 15;
        const int r0 = 32 * eh + 4 * g + (i16 >> 2);
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
        u32x4 va = vt_operand(0);
#pragma unroll
        for (int v = 0; v < VT; ++v) {
            if (v < vtiles) {
                u32x4 vn = va;
                if (v + 1 < vtiles) vn = vt_operand(v + 1);
                acc[v] = mfma16(va, pb, acc[v]);
                va = vn;
            }
        }
    };
    for (int blk = 0; blk < nblk; blk += 2) {
        run_block(blk, kvbuf0, kvbuf1);
        if (blk + 1 < nblk) run_block(blk + 1, kvbuf1, kvbuf0);
    }

    // ---- merge the two entry halves through LDS (reusing the KV buffers)
    float l_tot = l_run;
    l_tot += __shfl_xor(l_tot, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    __syncthreads();  // all waves done with the KV buffers
    float* xch = reinterpret_cast<float*>(kvbuf0) + (wave & 1) * (VT * 4 + 2) * 64;
    if (eh == 1) {
#pragma unroll
        for (int v = 0; v < VT; ++v)
#pragma unroll
            for (int j = 0; j < 4; ++j) xch[(v * 4 + j) * 64 + lane] = acc[v][j];
        xch[VT * 4 * 64 + lane] = m_run;
        xch[(VT * 4 + 1) * 64 + lane] = l_tot;
    }
    __syncthreads();
    if (eh == 1 || !head_ok) return;
    const float m_b = xch[VT * 4 * 64 + lane];
    const float l_b = xch[(VT * 4 + 1) * 64 + lane];
    const float M = fmaxf(m_run, m_b);
    const float sk = sink ? sink[head] * kLog2e : -INFINITY;
    float fa = 0.f, fb = 0.f, inv = 0.f, den = 0.f;
    if (M != -INFINITY) {
        fa = exp2f(m_run - M);
        fb = exp2f(m_b - M);
        den = l_tot * fa + l_b * fb + exp2f(sk - M);
        inv = 1.f / den;
        fa *= inv;
        fb *= inv;
    }
    uint16_t* orow = out + ((size_t)tok * Hq + head) * Dv;
#pragma unroll
    for (int v = 0; v < VT; ++v) {
        if (v < vtiles) {
            float o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = acc[v][j] * fa + xch[(v * 4 + j) * 64 + lane] * fb;
            uint2 w;
            w.x = pack_bf16x2(o[0], o[1]);
            w.y = pack_bf16x2(o[2], o[3]);
            *reinterpret_cast<uint2*>(orow + 16 * v + 4 * g) = w;
        }
    }
    if (lse && g == 0) {
        float val;
        if (M == -INFINITY) val = sink ? sink[head] : -INFINITY;
        else val = (M + log2f(den)) / kLog2e;
        lse[(size_t)tok * Hq + head] = val;
    }
}

template <int KSTEPS, int VT, int ROWU, bool EXACT>
hipError_t launch_variant(const void* q, const void* kv, const float* attn_sink, const int32_t* idx, int32_t B,
                          int32_t S, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t S_kv, int32_t K_top, float sm_scale,
                          void* out, float* lse, hipStream_t stream)
{
    const int BS = B * S;
    const int HG = (Hq + kHeadsPerGroup - 1) / kHeadsPerGroup;
    const int grid = (BS + kXcds - 1) / kXcds * kXcds * HG;
    sparse_attn_kernel<KSTEPS, VT, ROWU, EXACT><<<grid, kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv), attn_sink, idx, BS, S, Hq, Dqk, Dv, S_kv,
        K_top, sm_scale, static_cast<uint16_t*>(out), lse);
    return hipGetLastError();
}

}  // namespace

int sparse_attn_splits(int32_t, int32_t, int32_t, int32_t) { return 1; }

size_t sparse_attn_partial_bytes(int32_t, int32_t, int32_t, int32_t, int32_t) { return 0; }

hipError_t launch_sparse_attn(const void* q, const void* kv, const float* attn_sink, const int32_t* idx,
                              int32_t B, int32_t S, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t S_kv,
                              int32_t K_top, float sm_scale, void* out, float* lse, void*, hipStream_t stream)
{
    // Exact instances for the MLA decode shape (576 / 512) and the 192 / 128
    // shape; any other shape runs the predicated 576 / 512 instance.  ROWU
    // covers (Dqk / 8 + 1) | 1 for every Dqk an instance accepts.
    if (Dqk == 576 && Dv == 512)
        return launch_variant<18, 32, 73, true>(q, kv, attn_sink, idx, B, S, Hq, Dqk, Dv, S_kv, K_top, sm_scale, out,
                                                lse, stream);
    if (Dqk == 192 && Dv == 128)
        return launch_variant<6, 8, 25, true>(q, kv, attn_sink, idx, B, S, Hq, Dqk, Dv, S_kv, K_top, sm_scale, out,
                                              lse, stream);
    return launch_variant<18, 32, 73, false>(q, kv, attn_sink, idx, B, S, Hq, Dqk, Dv, S_kv, K_top, sm_scale, out,
                                             lse, stream);
}

}  // namespace dsa
