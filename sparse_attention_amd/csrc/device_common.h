// Device helpers shared by the gfx950 kernels of libdsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa_internal.h"

namespace dsa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Most negative finite bfloat16 (0xFF7F), exact in fp32: the finite mask
// bound of slots a row cannot attend to.
__host__ __device__ __forceinline__ float mask_bound() { return -0x1.FEp+127f; }

// Attendable slots of row r (positions+1, capped by valid_len, clamped).
__device__ __forceinline__ int n_valid_of(const int32_t* positions, int32_t valid_len, int32_t r, int32_t S_max)
{
    long long n = positions ? (long long)positions[r] + 1 : (long long)S_max;
    if (valid_len >= 0 && (long long)valid_len < n) n = valid_len;
    if (n < 0) n = 0;
    if (n > S_max) n = S_max;
    return (int)n;
}

// Same as n_valid_of in 32-bit arithmetic (cheaper when evaluated on the scalar unit).
__device__ __forceinline__ int n_valid_of32(const int32_t* positions, int32_t valid_len, int32_t r, int32_t S_max)
{
    int n = S_max;
    if (positions) {
        const int p = positions[r];
        n = p < S_max ? p + 1 : S_max;  // no overflow: p + 1 <= S_max
    }
    if (valid_len >= 0 && valid_len < n) n = valid_len;
    return n < 0 ? 0 : n;
}

// The two bfloat16 halves of a 32-bit word as fp32 (low half = lower address).
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// fp32 -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    // one v_cvt_pk_bf16_f32 on gfx950 (round to nearest even, as f32_to_bf16_bits)
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// DPP lane exchanges inside a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_QUAD_XOR1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

// Sum over the 16 lanes of a DPP row; every lane of the row gets the sum.
__device__ __forceinline__ float row16_sum(float x)
{
    x += dpp<DPP_QUAD_XOR1>(x);
    x += dpp<DPP_QUAD_XOR2>(x);
    x += dpp<DPP_ROW_HALF_MIRROR>(x);
    x += dpp<DPP_ROW_MIRROR>(x);
    return x;
}
// Sum over aligned groups of 8 lanes.
__device__ __forceinline__ float row8_sum(float x)
{
    x += dpp<DPP_QUAD_XOR1>(x);
    x += dpp<DPP_QUAD_XOR2>(x);
    x += dpp<DPP_ROW_HALF_MIRROR>(x);
    return x;
}

// Order-preserving map of a (non-NaN) fp32 to uint32: a < b  <=>  key(a) < key(b).
__device__ __forceinline__ uint32_t f32_order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Where slot s of sequence r lives in a key or KV store: row r * S_max + s of
// a contiguous [n_seq, S_max] store, or, for a page pool, row
// page * P + (s mod P) with page = block_table[r][s / P] (P = 2^lp slots per
// page).  A page id outside [0, n_pages) is clamped into the pool, so a bad
// table reads wrong rows but never leaves the allocation.
template <bool PAGED>
__device__ __forceinline__ size_t store_row(const PageMap& pm, int r, int s, int S_max)
{
    if (!PAGED) return (size_t)r * S_max + s;
    // callers may ask for slots past the sequence's last page (rounds that load
    // nothing): the table column is clamped too, so the table read stays in bounds
    const int col = min(s >> pm.lp, pm.max_pages - 1);
    const uint32_t page = min((uint32_t)pm.table[(size_t)r * pm.max_pages + col], (uint32_t)(pm.n_pages - 1));
    return ((size_t)page << pm.lp) | (uint32_t)(s & ((1 << pm.lp) - 1));
}

// Grid-stride clear of an unrelated buffer riding along with a 2-D launch
// (saves the stream a launch of its own).
__device__ __forceinline__ void clear_words(uint32_t* __restrict__ p, size_t n)
{
    if (!n) return;
    const size_t wg = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
    const size_t stride = (size_t)gridDim.x * gridDim.y * blockDim.x;
    for (size_t i = wg * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

}  // namespace dsa
