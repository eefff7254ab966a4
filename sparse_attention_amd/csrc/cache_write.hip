// Key-cache write with FP8 block quantisation, for gfx950.
//
// Definition ([NKI-V32] key_cache: the cache is written in place at each
// token's current position; [V4-KERNEL] FP8 block quantisation: blocks of
// 128 elements, scale = amax / 448 so the block fits E4M3's +-448, optional
// power-of-two scale, optional quantise-then-dequantise to bfloat16):
//   token t goes to cache row t / rows_per_seq, slot positions[t] (skipped
//   when outside [0, S_max)); for fp8, s = amax / 448 (1 for an all-zero
//   block; with the power-of-two option the smallest 2^e >= it), the codes
//   are the nearest E4M3 values of clamp(k / s, -448, 448), ties to even,
//   and the slot's scale is s.
//
// Every decision that picks a code is one binary32 operation: the amax is
// exact, amax / 448 and k / s are IEEE divisions (hipcc's default float
// division is correctly rounded), the clamp is exact, and
// v_cvt_pk_fp8_f32 rounds to nearest even.  The codes are therefore those
// of any exact binary32 implementation, bit for bit.
//
// The work is a few hundred bytes per token, so the kernel is bound by
// launch latency at decode sizes and by HBM at prefill sizes:
//   * 16 lanes per token, 8 elements (one 16-byte load) per lane, so a wave
//     moves 4 tokens = 1 KiB of keys with one load instruction;
//   * the amax is a DPP max over the 16-lane row;
//   * fp8: 8 codes per lane go out as one 8-byte store (128 contiguous bytes
//     per token) and lane 0 of the row stores the scale;
//   * bf16: one 16-byte store per lane;
//   * paged caches: the slot's pool row comes from the block table.
#include "device_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;
constexpr int kTokPerWg = kThreads / 16;

__device__ __forceinline__ float row16_max(float x)
{
    x = fmaxf(x, dpp<DPP_QUAD_XOR1>(x));
    x = fmaxf(x, dpp<DPP_QUAD_XOR2>(x));
    x = fmaxf(x, dpp<DPP_ROW_HALF_MIRROR>(x));
    x = fmaxf(x, dpp<DPP_ROW_MIRROR>(x));
    return x;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// MODE 0: fp8 codes + scale; 1: bf16 copy; 2: bf16 quantised and dequantised.
// PAGED: k_cache / k_scale are page pools addressed through pm.
template <int MODE, bool PAGED>
__global__ __launch_bounds__(kThreads) void cache_write_kernel(const uint16_t* __restrict__ k_new, int32_t T,
                                                               int32_t rows_per_seq,
                                                               const int32_t* __restrict__ positions,
                                                               uint8_t* __restrict__ k_cache,
                                                               float* __restrict__ k_scale, int32_t S_max,
                                                               bool round_scale, PageMap pm)
{
    const int t = blockIdx.x * kTokPerWg + (threadIdx.x >> 4);
    const int e = threadIdx.x & 15;  // elements 8 e .. 8 e + 7
    // rows of 16 lanes stay together through the DPP reduction, so a row
    // whose token is out of range or skipped leaves as a whole
    if (t >= T) return;
    const int p = positions[t];
    if (p < 0 || p >= S_max) return;
    const size_t slot = store_row<PAGED>(pm, t / rows_per_seq, p, S_max);

    const u32x4 v = *reinterpret_cast<const u32x4*>(k_new + (size_t)t * 128 + 8 * e);
    if (MODE == 1) {
        *reinterpret_cast<u32x4*>(k_cache + slot * 256 + 16 * e) = v;
        return;
    }
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_bits_to_f32(v[i] & 0xFFFFu);
        x[2 * i + 1] = bf16_bits_to_f32(v[i] >> 16);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = row16_max(amax);

    float s = 1.f;
    if (amax > 0.f) {
        s = amax / 448.f;
        if (round_scale) {
            int ex;
            const float m = frexpf(s, &ex);  // s = m 2^ex, m in [0.5, 1)
            if (m != 0.5f) s = ldexpf(1.f, ex);
        }
    }
    uint32_t codes[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = fminf(fmaxf(x[4 * i + j] / s, -448.f), 448.f);
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
        codes[i] = (uint32_t)w;
    }
    if (MODE == 0) {
        *reinterpret_cast<uint2*>(k_cache + slot * 128 + 8 * e) = make_uint2(codes[0], codes[1]);
        if (e == 0) k_scale[slot] = s;
    } else {
        // exact decode of the codes (bytes 0,1 and 2,3 of each word), then
        // one binary32 product and one rounding to bfloat16
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes[i], false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes[i], true);
            o[2 * i] = pack_bf16x2(lo[0] * s, lo[1] * s);
            o[2 * i + 1] = pack_bf16x2(hi[0] * s, hi[1] * s);
        }
        *reinterpret_cast<u32x4*>(k_cache + slot * 256 + 16 * e) = o;
    }
}

}  // namespace

hipError_t launch_cache_write(const void* k_new, int32_t T, int32_t rows_per_seq, const int32_t* positions,
                              bool key_fp8, bool qdq, bool round_scale, void* k_cache, float* k_scale,
                              int32_t S_max, const PageMap* paging, hipStream_t stream)
{
    if (T == 0) return hipSuccess;
    const dim3 grid((T + kTokPerWg - 1) / kTokPerWg);
    const auto* kn = static_cast<const uint16_t*>(k_new);
    auto* kc = static_cast<uint8_t*>(k_cache);
    const PageMap pm = paging ? *paging : PageMap{nullptr, 0, 0, 0};
#define DSA_CW_LAUNCH(MODE, KS, RS)                                                                                \
    (paging ? cache_write_kernel<MODE, true><<<grid, kThreads, 0, stream>>>(kn, T, rows_per_seq, positions, kc, KS, \
                                                                            S_max, RS, pm)                         \
            : cache_write_kernel<MODE, false><<<grid, kThreads, 0, stream>>>(kn, T, rows_per_seq, positions, kc, KS, \
                                                                             S_max, RS, pm))
    if (key_fp8)
        DSA_CW_LAUNCH(0, k_scale, round_scale);
    else if (qdq)
        DSA_CW_LAUNCH(2, nullptr, round_scale);
    else
        DSA_CW_LAUNCH(1, nullptr, false);
#undef DSA_CW_LAUNCH
    return hipGetLastError();
}

}  // namespace dsa
