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
//   * workgroup = (query token, 64-head group, split of the index list);
//     4 waves x 16 heads; MFMA v_mfma_f32_16x16x32_bf16.
//   * gather: the 64 listed KV rows of a block are loaded (16 B per lane,
//     128-B row segments) and stored in LDS "pair-interleaved": word
//     [p][d] holds (kv[row 2p][d], kv[row 2p + 1][d]) as two bf16.  Masked
//     rows are stored as zeros.  One layout serves both contractions:
//       - QK^T (contracts over d): M = entries, split into an even-row and
//         an odd-row tile; a lane reads 8 consecutive words (32 B) of one
//         pair and unpacks the even and odd A operands from them;  B = q,
//         held in registers for the whole kernel;
//       - P.V (contracts over entries): the even/odd S tiles in the MFMA
//         accumulator layout are exactly the B operand (P^T, N = heads) of
//         a 32-entry K step, and the A operand (V^T, M = value dims) is 4
//         words [p][v] of consecutive pairs -- no transpose anywhere.
//   * softmax state (max, partial sum) per head lives in registers, in
//     log2 units (exp2); output accumulators O^T[v][head] in registers.
//   * the index list is split across workgroups when there are too few
//     (token, head group) pairs to fill the chip; partial (max, sum, O) go
//     to the workspace and a combine kernel merges them and adds the sink.
#include "device_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kHeadsPerWave = 16;
constexpr int kHeadsPerGroup = 64;
constexpr int kBlock = 64;          // index-list entries per block
constexpr int kPairs = kBlock / 2;  // 32
constexpr int kMaxDqk = 576;
constexpr int kRowWords = kMaxDqk + 4;  // padded pair-row length in 32-bit words
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t dpp_xor1_u32(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, DPP_QUAD_XOR1, 0xF, 0xF, false);
}

// KSTEPS: max Dqk / 32 held in registers; VT: max Dv / 16 value tiles.
template <int KSTEPS, int VT>
__global__ __launch_bounds__(kThreads, 2) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const float* __restrict__ sink,
    const int32_t* __restrict__ idx, int32_t S, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t S_kv, int32_t K_top,
    float sm_scale, int32_t n_split, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_ml)
{
    __shared__ __attribute__((aligned(16))) uint32_t kvs[kPairs * kRowWords];
    __shared__ int sidx[kBlock];

    const int split = blockIdx.x;
    const int hgrp = blockIdx.y;
    const int bs = blockIdx.z;  // b * S + s
    const int b = bs / S;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;   // MFMA column: head within the wave
    const int g = lane >> 4;   // MFMA lane group
    const int head = hgrp * kHeadsPerGroup + wave * kHeadsPerWave + n;
    const bool head_ok = head < Hq;
    const int ksteps = Dqk / 32;
    const int vtiles = Dv / 16;

    // q of this lane's head: B operand of QK^T, dims 32t + 8g .. +7 per K step
    u32x4 qreg[KSTEPS];
    {
        const uint16_t* qh = q + ((size_t)bs * Hq + (head_ok ? head : 0)) * Dqk + 8 * g;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t)
            qreg[t] = (head_ok && t < ksteps) ? *reinterpret_cast<const u32x4*>(qh + 32 * t) : u32x4{0, 0, 0, 0};
    }

    f32x4 acc[VT];
#pragma unroll
    for (int v = 0; v < VT; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;  // running max, log2 units
    float l_run = 0.f;        // this lane's share of the running sum

    const float qk_scale = sm_scale * kLog2e;
    const int nblocks = (K_top + kBlock - 1) / kBlock;
    const int per = nblocks / n_split, extra = nblocks % n_split;
    const int blk0 = split * per + min(split, extra);
    const int blk1 = blk0 + per + (split < extra ? 1 : 0);
    const int32_t* __restrict__ ilist = idx + (size_t)bs * K_top;
    const uint16_t* __restrict__ kvb = kv + (size_t)b * S_kv * Dqk;

    // gather lane roles: 4 pairs x 8 chunks x 2 rows per wave instruction
    const int gpar = lane & 1;
    const int gchunk = (lane >> 1) & 7;
    const int gpair = (lane >> 4) + 4 * wave;  // 0..15
    const int nchunks = Dqk / 8;

    for (int blk = blk0; blk < blk1; ++blk) {
        __syncthreads();  // previous block fully consumed
        if (threadIdx.x < kBlock) {
            const int j = blk * kBlock + threadIdx.x;
            int t = j < K_top ? ilist[j] : -1;
            sidx[threadIdx.x] = (t >= 0 && t < S_kv) ? t : -1;
        }
        __syncthreads();
        // ---- gather into the pair-interleaved layout
        for (int p0 = 0; p0 < kPairs; p0 += 16) {
            const int p = p0 + gpair;
            const int row = sidx[2 * p + gpar];
            for (int c0 = 0; c0 < nchunks; c0 += 8) {
                const int c = c0 + gchunk;
                u32x4 v = {0, 0, 0, 0};
                if (c < nchunks && row >= 0) v = *reinterpret_cast<const u32x4*>(kvb + (size_t)row * Dqk + 8 * c);
                // even lane keeps dims 0..3 of its row and receives the odd row's;
                // odd lane keeps dims 4..7 of its row and receives the even row's.
                const uint32_t s0 = gpar ? v[0] : v[2];
                const uint32_t s1 = gpar ? v[1] : v[3];
                const uint32_t r0 = dpp_xor1_u32(s0);
                const uint32_t r1 = dpp_xor1_u32(s1);
                const uint32_t e0 = gpar ? r0 : v[0], e1 = gpar ? r1 : v[1];  // even row words
                const uint32_t o0 = gpar ? v[2] : r0, o1 = gpar ? v[3] : r1;  // odd row words
                if (c < nchunks) {
                    u32x4 wv;
                    wv[0] = lo_pair(e0, o0);
                    wv[1] = hi_pair(e0, o0);
                    wv[2] = lo_pair(e1, o1);
                    wv[3] = hi_pair(e1, o1);
                    *reinterpret_cast<u32x4*>(&kvs[p * kRowWords + 8 * c + 4 * gpar]) = wv;
                }
            }
        }
        __syncthreads();

        // ---- S = KV . q^T : tiles [chunk][parity], rows = pairs 16c + 4g + j
        f32x4 sacc[2][2];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int par = 0; par < 2; ++par) sacc[c][par] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            if (t < ksteps) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const uint32_t* src = &kvs[(16 * c + n) * kRowWords + 32 * t + 8 * g];
                    const u32x4 w0 = *reinterpret_cast<const u32x4*>(src);
                    const u32x4 w1 = *reinterpret_cast<const u32x4*>(src + 4);
                    const u32x4 ae = {lo_pair(w0[0], w0[1]), lo_pair(w0[2], w0[3]), lo_pair(w1[0], w1[1]),
                                      lo_pair(w1[2], w1[3])};
                    const u32x4 ao = {hi_pair(w0[0], w0[1]), hi_pair(w0[2], w0[3]), hi_pair(w1[0], w1[1]),
                                      hi_pair(w1[2], w1[3])};
                    sacc[c][0] = mfma16(ae, qreg[t], sacc[c][0]);
                    sacc[c][1] = mfma16(ao, qreg[t], sacc[c][1]);
                }
            }
        }

        // ---- online softmax (log2 units); entry of (c, par, j) = 32c + 8g + 2j + par
        float sv[2][2][4];
        float bmax = -INFINITY;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int par = 0; par < 2; ++par)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bool ok = sidx[32 * c + 8 * g + 2 * j + par] >= 0;
                    const float x = ok ? sacc[c][par][j] * qk_scale : -INFINITY;
                    sv[c][par][j] = x;
                    bmax = fmaxf(bmax, x);
                }
        bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
        bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
        const float m_new = fmaxf(m_run, bmax);
        const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
        const float msub = (m_new == -INFINITY) ? 0.f : m_new;
        float psum = 0.f;
        u32x4 pb[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            float pe[4], po[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pe[j] = exp2f(sv[c][0][j] - msub);
                po[j] = exp2f(sv[c][1][j] - msub);
                psum += pe[j] + po[j];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) pb[c][j] = pack_bf16x2(pe[j], po[j]);
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int v = 0; v < VT; ++v) acc[v] *= alpha;

        // ---- O^T += V^T . P^T : A = 4 words [16c + 4g + i][v], B = pb[c]
#pragma unroll
        for (int v = 0; v < VT; ++v) {
            if (v < vtiles) {
                const int col = 16 * v + n;
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const uint32_t* src = &kvs[(16 * c + 4 * g) * kRowWords + col];
                    const u32x4 a = {src[0], src[kRowWords], src[2 * kRowWords], src[3 * kRowWords]};
                    acc[v] = mfma16(a, pb[c], acc[v]);
                }
            }
        }
    }

    // ---- epilogue: lane (head n, group g) holds O^T[16v + 4g + j][head]
    float l_tot = l_run;
    l_tot += __shfl_xor(l_tot, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    if (!head_ok) return;
    if (n_split == 1) {
        const float sk = sink ? sink[head] * kLog2e : -INFINITY;
        float den, inv;
        if (m_run == -INFINITY) {
            den = 0.f;
            inv = 0.f;
        } else {
            den = l_tot + exp2f(sk - m_run);
            inv = 1.f / den;
        }
        uint16_t* orow = out + ((size_t)bs * Hq + head) * Dv;
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
            lse[(size_t)bs * Hq + head] = val;
        }
    } else {
        const size_t item = ((size_t)split * gridDim.z + bs) * Hq + head;
        float* po = part_o + item * Dv;
#pragma unroll
        for (int v = 0; v < VT; ++v)
            if (v < vtiles) *reinterpret_cast<f32x4*>(po + 16 * v + 4 * g) = acc[v];
        if (g == 0) {
            part_ml[2 * item] = m_run;
            part_ml[2 * item + 1] = l_tot;
        }
    }
}

// Merge split partials: M = max m_i, den = sum l_i 2^(m_i - M) + 2^(sink - M),
// out = sum O_i 2^(m_i - M) / den.  One workgroup per (token, head).
__global__ __launch_bounds__(128) void sparse_attn_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, const float* __restrict__ sink,
    int32_t n_split, int32_t n_items, int32_t Hq, int32_t Dv, uint16_t* __restrict__ out, float* __restrict__ lse)
{
    const int item = blockIdx.x;  // bs * Hq + head
    const int head = item % Hq;
    float M = -INFINITY;
    for (int i = 0; i < n_split; ++i) M = fmaxf(M, part_ml[2 * ((size_t)i * n_items + item)]);
    const float sk = sink ? sink[head] * kLog2e : -INFINITY;
    float den = 0.f;
    if (M != -INFINITY) {
        for (int i = 0; i < n_split; ++i) {
            const size_t it = (size_t)i * n_items + item;
            den += part_ml[2 * it + 1] * exp2f(part_ml[2 * it] - M);
        }
        den += exp2f(sk - M);
    }
    const float inv = (M == -INFINITY) ? 0.f : 1.f / den;
    for (int v = threadIdx.x; v < Dv; v += blockDim.x) {
        float o = 0.f;
        if (M != -INFINITY)
            for (int i = 0; i < n_split; ++i) {
                const size_t it = (size_t)i * n_items + item;
                const float m_i = part_ml[2 * it];
                if (m_i != -INFINITY) o += part_o[it * Dv + v] * exp2f(m_i - M);
            }
        out[(size_t)item * Dv + v] = (uint16_t)f32_to_bf16_bits(o * inv);
    }
    if (lse && threadIdx.x == 0) {
        float val;
        if (M == -INFINITY) val = sink ? sink[head] : -INFINITY;
        else val = (M + log2f(den)) / kLog2e;
        lse[item] = val;
    }
}

constexpr int kTargetWorkgroups = 512;  // ~2 resident per CU on 256 CUs

}  // namespace

int sparse_attn_splits(int32_t B, int32_t S, int32_t Hq, int32_t K_top)
{
    const long long base = (long long)B * S * ((Hq + kHeadsPerGroup - 1) / kHeadsPerGroup);
    const int nblocks = (K_top + kBlock - 1) / kBlock;
    long long want = (kTargetWorkgroups + base - 1) / base;
    if (want > nblocks) want = nblocks;
    if (want < 1) want = 1;
    return (int)want;
}

size_t sparse_attn_partial_bytes(int32_t B, int32_t S, int32_t Hq, int32_t Dv, int32_t K_top)
{
    const int ns = sparse_attn_splits(B, S, Hq, K_top);
    if (ns <= 1) return 0;
    return (size_t)ns * B * S * Hq * ((size_t)Dv + 2) * sizeof(float);
}

hipError_t launch_sparse_attn(const void* q, const void* kv, const float* attn_sink, const int32_t* idx,
                              int32_t B, int32_t S, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t S_kv,
                              int32_t K_top, float sm_scale, void* out, float* lse, void* workspace,
                              hipStream_t stream)
{
    const int ns = sparse_attn_splits(B, S, Hq, K_top);
    const int n_items = B * S * Hq;
    float* part_o = nullptr;
    float* part_ml = nullptr;
    if (ns > 1) {
        part_o = static_cast<float*>(workspace);
        part_ml = part_o + (size_t)ns * n_items * Dv;
    }
    const dim3 grid(ns, (Hq + kHeadsPerGroup - 1) / kHeadsPerGroup, B * S);
    const auto* qp = static_cast<const uint16_t*>(q);
    const auto* kvp = static_cast<const uint16_t*>(kv);
    auto* op = static_cast<uint16_t*>(out);
    if (Dqk <= 192 && Dv <= 128)
        sparse_attn_kernel<6, 8><<<grid, kThreads, 0, stream>>>(qp, kvp, attn_sink, idx, S, Hq, Dqk, Dv, S_kv, K_top,
                                                                sm_scale, ns, op, lse, part_o, part_ml);
    else
        sparse_attn_kernel<18, 32><<<grid, kThreads, 0, stream>>>(qp, kvp, attn_sink, idx, S, Hq, Dqk, Dv, S_kv,
                                                                  K_top, sm_scale, ns, op, lse, part_o, part_ml);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ns <= 1) return e;
    sparse_attn_combine_kernel<<<n_items, 128, 0, stream>>>(part_o, part_ml, attn_sink, ns, n_items, Hq, Dv, op, lse);
    return hipGetLastError();
}

}  // namespace dsa
