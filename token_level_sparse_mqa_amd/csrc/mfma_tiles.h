// Shared pieces of the MFMA attention kernels (gfx950): operand types, FP8 conversion, and the
// LDS tile of 32 cache rows that every MFMA kernel stages K and V through.
//
// Global -> registers: a 32-row tile is read with coalesced 16-byte loads, each wave load
// instruction covering whole rows (1 KB of consecutive bytes).  Registers -> LDS: rows are
// stored as bf16 (FP8 codes are converted exactly on the way), with the 16-byte chunks of row
// r XOR-swizzled by r so that MFMA operand reads, which take the same chunk of 32 different
// rows, spread over the LDS banks.  V is read back transposed with ds_read_b64_tr_b16.
#pragma once

#include "hs2_device.h"

namespace hs2 {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

constexpr int kTileRows = 32;

// ---- conversions ---------------------------------------------------------------------------------

// Two E4M3FN codes (bytes 0/1 or 2/3 of w) -> two fp32, exact.
template <bool HI>
__device__ __forceinline__ f32x2_t fp8x2_to_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// Four E4M3 codes (one dword) -> four bf16 (two dwords), one conversion per pair.  bf16 holds
// every E4M3 value exactly, so with scale 1 the result is the code's value.
__device__ __forceinline__ u32x2_t fp8x4_to_bf16x4(uint32_t w) {
    u32x2_t r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
    return r;
}

// fp32 -> bf16 hi + bf16 lo with hi + lo = x to about 2^-16 relative.
__device__ __forceinline__ void split_bf16x8(const float* x, bf16x8_t& hi, bf16x8_t& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 h = (__bf16)x[e];
        hi[e] = h;
        lo[e] = (__bf16)(x[e] - (float)h);
    }
}

__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// ---- the LDS tile: 32 rows of D 16-bit values ---------------------------------------------------
// K tiles are read as 16-byte row chunks by 32 lanes at a time (chunk XOR row spreads them over
// the banks).  V tiles are read transposed: the two 16-lane groups of a half wave read the same
// 4 consecutive rows, each group one pair of adjacent chunks per row, the second group's pair 2
// chunks after the first's.  At D = 128 the chunk is XORed with 4 (row mod 4) + 2 ((row / 4) mod 2):
// bit 1 of the XOR is the same for the 4 rows, so the 8 chunk pairs of the two groups land in 8
// different bank groups.  At D = 64 (8 chunks a row) the XOR 2 (row mod 4) keeps each group free
// of conflicts.  Any per-row XOR leaves the row-wise stores free of conflicts.
template <int D>
struct LdsTile {
    static constexpr int RB = D * 2;          // bytes per row
    static constexpr int CPR = D / 8;         // 16-byte chunks per row
    static constexpr int BYTES = kTileRows * RB;
    __device__ static __forceinline__ int off(int row, int chunk) {
        return row * RB + ((chunk ^ (row & (CPR - 1))) << 4);
    }
    __device__ static __forceinline__ int vswz(int row) {
        return CPR >= 16 ? (((row & 3) << 2) | (((row >> 2) & 1) << 1)) : ((row << 1) & (CPR - 2));
    }
    __device__ static __forceinline__ int voff(int row, int chunk) {
        return row * RB + ((chunk ^ vswz(row)) << 4);
    }
};

// Geometry of the coalesced global loads of a 32-row tile in storage format.
template <int D, int KV>
struct RawGeom {
    static constexpr int ESZ = KV == HS2_FP8_E4M3 ? 1 : 2;
    static constexpr int RB = D * ESZ;        // bytes per stored row
    static constexpr int CPR = RB / 16;       // 16-byte chunks per stored row
    static constexpr int RPI = 64 / CPR;      // rows per wave load instruction
    static constexpr int NI = kTileRows / RPI;  // load instructions per tile
};

// 16-byte load; NT = non-temporal (the line is not kept in the caches for reuse).
template <bool NT>
__device__ __forceinline__ u32x4_t ld16(const void* p) {
    if constexpr (NT) return __builtin_nontemporal_load((const u32x4_t*)p);
    else return *(const u32x4_t*)p;
}

// Issue the NI coalesced loads of a tile: lane l of instruction x reads chunk l % CPR of tile
// row RPI*x + l / CPR, whose cache row index is src_row(tile row).
template <int D, int KV, bool NT, class RowFn>
__device__ __forceinline__ void load_raw_tile(u32x4_t* raw, const void* base, RowFn src_row) {
    using G = RawGeom<D, KV>;
    const int lane = threadIdx.x & 63;
    const int c = lane % G::CPR;
#pragma unroll
    for (int x = 0; x < G::NI; ++x) {
        const int R = G::RPI * x + lane / G::CPR;
        const int64_t row = src_row(R);
        raw[x] = ld16<NT>((const char*)base + row * G::RB + 16 * c);
    }
}

// Store a raw tile into the LDS tile as bf16 (rows with keep(R) == false become zero), in the
// K layout or (VT = true) the V layout.
template <int D, int KV, bool VT, class KeepFn>
__device__ __forceinline__ void store_lds_tile(const u32x4_t* raw, char* lds, KeepFn keep) {
    using G = RawGeom<D, KV>;
    using T = LdsTile<D>;
    auto off = [](int row, int chunk) { return VT ? T::voff(row, chunk) : T::off(row, chunk); };
    const int lane = threadIdx.x & 63;
    const int c = lane % G::CPR;
#pragma unroll
    for (int x = 0; x < G::NI; ++x) {
        const int R = G::RPI * x + lane / G::CPR;
        const uint32_t msk = keep(R) ? 0xffffffffu : 0u;
        if (KV == HS2_FP8_E4M3) {
            // 16 codes -> 16 bf16 = two LDS chunks
            u32x4_t lo, hi;
            const u32x2_t a = fp8x4_to_bf16x4(raw[x][0] & msk), b = fp8x4_to_bf16x4(raw[x][1] & msk);
            const u32x2_t cc = fp8x4_to_bf16x4(raw[x][2] & msk), d = fp8x4_to_bf16x4(raw[x][3] & msk);
            lo[0] = a[0]; lo[1] = a[1]; lo[2] = b[0]; lo[3] = b[1];
            hi[0] = cc[0]; hi[1] = cc[1]; hi[2] = d[0]; hi[3] = d[1];
            *(u32x4_t*)(lds + off(R, 2 * c)) = lo;
            *(u32x4_t*)(lds + off(R, 2 * c + 1)) = hi;
        } else {
            u32x4_t v = raw[x];
            v[0] &= msk; v[1] &= msk; v[2] &= msk; v[3] &= msk;
            *(u32x4_t*)(lds + off(R, c)) = v;
        }
    }
}

// MFMA operand with 8 consecutive d of tile row `row`: d in [8 * chunk, 8 * chunk + 8).
template <int D>
__device__ __forceinline__ bf16x8_t lds_row_operand(const char* lds, int row, int chunk) {
    return *(const bf16x8_t*)(lds + LdsTile<D>::off(row, chunk));
}

// A operand of O^T[dv][head] += V^T . P^T for dv block `blk` (32 dims) and k-step `ks`
// (16 keys): lane (m = dv - 32 blk, hb) receives V[key][dv] for keys 16ks + 4hb + {0..3} and
// 16ks + 8 + 4hb + {0..3}.  ds_read_b64_tr_b16 transposes within each 16-lane group: source
// lane q of the group supplies 4 consecutive dims of key row (q >> 2), and result lane i gets
// element i of each of the four rows.
template <int D>
__device__ __forceinline__ bf16x8_t lds_vt_operand(const char* lds, int blk, int ks) {
    const int lane = threadIdx.x & 63;
    const int G = lane >> 4, q = lane & 15;
    const int hb = G >> 1;
    const int dv = blk * 32 + 16 * (G & 1) + 4 * (q & 3);
    u32x4_t r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int key = 16 * ks + 8 * h + 4 * hb + (q >> 2);
        const char* p = lds + LdsTile<D>::voff(key, dv >> 3) + (dv & 7) * 2;
        const v4i16_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)p);
        const u32x2_t tu = __builtin_bit_cast(u32x2_t, t);
        r[2 * h] = tu[0];
        r[2 * h + 1] = tu[1];
    }
    return __builtin_bit_cast(bf16x8_t, r);
}

}  // namespace hs2
