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

__device__ __forceinline__ float wave_max(float x) {
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    const int lane = threadIdx.x & 63;
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    return x;
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
