// Device-side helpers shared by the hs2 kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hs2_internal.h"

namespace hs2 {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();

// ---- number formats ------------------------------------------------------------------------

// bfloat16 is the upper half of a binary32.
__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// binary32 -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// OCP FP8 E4M3FN code -> binary32 (exact).  Exponent field 0: m * 2^-9; S.1111.111: NaN;
// otherwise (1 + m/8) * 2^(e-7), i.e. the 7 low bits shifted into a binary32 with the
// exponent re-biased from 7 to 127.
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t c) {
    const uint32_t em = c & 0x7fu;
    float v = (em >= 0x08u) ? __uint_as_float((em << 20) + ((127u - 7u) << 23)) : (float)em * 0.001953125f;
    v = (em == 0x7fu) ? __builtin_nanf("") : v;
    return __uint_as_float(__float_as_uint(v) | ((c & 0x80u) << 24));
}

// Element e of a cache row stored as dtype `dt`.
__device__ __forceinline__ float load_elem(const void* base, int dt, int64_t e) {
    if (dt == HS2_F32) return ((const float*)base)[e];
    if (dt == HS2_BF16) return bf16_to_f32(((const uint16_t*)base)[e]);
    return e4m3fn_to_f32(((const uint8_t*)base)[e]);
}

// ---- query rows ----------------------------------------------------------------------------

// Number of visible cache rows of sequence b.
__device__ __forceinline__ int64_t seq_len(const int32_t* kv_len, int b, int64_t Nmax) {
    if (!kv_len) return Nmax;
    int64_t L = kv_len[b];
    return L < 0 ? 0 : (L > Nmax ? Nmax : L);
}

// Position of query row r, or -1 when it is outside [0, len).
__device__ __forceinline__ int64_t row_pos(const int32_t* q_pos, const int32_t* kv_len, int r, int Tq,
                                           int64_t Nmax) {
    const int b = r / Tq;
    const int64_t t = q_pos[r];
    const int64_t L = seq_len(kv_len, b, Nmax);
    return (t >= 0 && t < L) ? t : -1;
}

// Global candidates of a row at position t: j in [0, t - window].
__device__ __forceinline__ int64_t cand_count(int64_t t, int window) {
    return t < 0 ? 0 : (t - window + 1 > 0 ? t - window + 1 : 0);
}

// ---- wave / block primitives ---------------------------------------------------------------

// Cross-lane steps stay in vector registers (DPP lane moves and the 16- and 32-lane swaps) rather
// than going through LDS permutes, whose round trips would chain up in these reductions and scans.
// DPP control words: row_shr:n = 0x110 + n, row_ror:n = 0x120 + n, row_bcast:15 = 0x142,
// row_bcast:31 = 0x143, quad_perm = four 2-bit lane selectors.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    // lanes without a source (or outside ROWS) read 0
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
// a, b: the values of lanes l and l ^ 16 (l ^ 32), in an order that depends on the lane; callers
// combine them symmetrically (max, or a sum, whose two operands commute exactly)
__device__ __forceinline__ void lane_pair16(float x, float& a, float& b) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(p[0]);
    b = __uint_as_float(p[1]);
}
__device__ __forceinline__ void lane_pair32(float x, float& a, float& b) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(p[0]);
    b = __uint_as_float(p[1]);
}

// Maximum / sum over the 64 lanes (every lane receives the maximum; the sum's rounding order
// can differ between lanes, so callers take it from one lane).  Within a 16-lane row a rotation by 8,
// one by 4 and two quad permutations combine all 16 lanes; the swaps then combine the rows.
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_f32<0x128>(x));
    x = fmaxf(x, dpp_f32<0x124>(x));
    x = fmaxf(x, dpp_f32<0x4E>(x));
    x = fmaxf(x, dpp_f32<0xB1>(x));
    float a, b;
    lane_pair16(x, a, b);
    lane_pair32(fmaxf(a, b), a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_f32<0x128>(x);
    x += dpp_f32<0x124>(x);
    x += dpp_f32<0x4E>(x);
    x += dpp_f32<0xB1>(x);
    float a, b;
    lane_pair16(x, a, b);
    lane_pair32(a + b, a, b);
    return a + b;
}

// Maximum over aligned groups of `group` lanes (a power of two up to 64, wave-uniform) of values
// that are >= 0 or negative markers that are all equal: each lane receives its group's maximum.
// Quad permutations pair lanes 1 and 2 apart, the half-row and row mirrors (0x141, 0x140) pair the
// 4-lane quads and the 8-lane halves of a 16-lane row, and the swaps pair the rows.  For such
// values the signed integer order of the bit patterns is the float order, so each step is one
// integer max (a float max costs three: the compiler canonicalises both operands first).
__device__ __forceinline__ float group_max_nonneg(float v, int group) {
    int x = __float_as_int(v);
    if (group >= 2) x = max(x, (int)dpp_u32<0xB1>((uint32_t)x));
    if (group >= 4) x = max(x, (int)dpp_u32<0x4E>((uint32_t)x));
    if (group >= 8) x = max(x, (int)dpp_u32<0x141>((uint32_t)x));
    if (group >= 16) x = max(x, (int)dpp_u32<0x140>((uint32_t)x));
    if (group >= 32) {
        const auto p = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
        x = max((int)p[0], (int)p[1]);
    }
    if (group >= 64) {
        const auto p = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
        x = max((int)p[0], (int)p[1]);
    }
    return __int_as_float(x);
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4 and 8 scan each 16-lane
// row, then the last lane of row 0 (row 2) is added to row 1 (row 3) and lane 31 to rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += dpp_u32<0x111>(x);
    x += dpp_u32<0x112>(x);
    x += dpp_u32<0x114>(x);
    x += dpp_u32<0x118>(x);
    x += dpp_u32<0x142, 0xA>(x);
    x += dpp_u32<0x143, 0xC>(x);
    return x;
}
// A lane's value broadcast to the wave (lane is wave-uniform).
__device__ __forceinline__ uint32_t lane_value(uint32_t x, int lane) {
    return (uint32_t)__builtin_amdgcn_readlane((int)x, lane);
}

// Exclusive block-wide prefix sum; `tmp` holds NT/64 + 1 words of LDS.  Returns the
// exclusive prefix of this thread; *total receives the block total.  All threads call it.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* tmp, uint32_t* total) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t inc = wave_incl_scan(x);
    if (lane == 63) tmp[w] = inc;
    __syncthreads();
    if (w == 0) {
        uint32_t v = lane < NW ? tmp[lane] : 0u;
        uint32_t vi = wave_incl_scan(v);
        if (lane < NW) tmp[lane] = vi - v;
        if (lane == NW - 1) tmp[NW] = vi;
    }
    __syncthreads();
    uint32_t res = tmp[w] + inc - x;
    *total = tmp[NW];
    __syncthreads();
    return res;
}

}  // namespace hs2
