// MFMA attention for one query row per workgroup (decode rows, sparse rows): device code.
//
// MQA (ainews page, experimental-setup paragraph): all H query heads of a token share one K/V
// row, so a 32-key tile of the cache is read once and multiplied against all heads with
// v_mfma_f32_32x32x16_bf16 (heads padded to 32 form the N dimension).  The full layer (causal
// range of keys) and the sparse layers (a list of selected rows: KV Reuse, lynxflow blog
// "Two-Level KV Sharing") share this kernel; only the source of the key ids differs.
//
// Per wave and 32-key tile (K and V staged through the wave's LDS tiles, see mfma_tiles.h):
//   S^T[key][head] = K_tile . Q^T          D/16 MFMAs; lane (n, hb) owns head n
//   online softmax per head in base 2      (x = s * sm * log2 e; 16 keys per lane + partner)
//   O^T[dv][head] += V^T . P^T             P split into bf16 hi + lo (two MFMAs per step)
// The four waves of a workgroup take interleaved tiles of the workgroup's key range and are
// merged in LDS; several workgroups per row (splits) are merged by attn_split_combine.
//
// The d order inside the QK product is free (both operands use it): lane half hb covers
// d in [hb*D/2, hb*D/2 + D/2), eight consecutive values per k-step.  The key order inside the
// PV product follows the S^T register layout, so P needs no shuffles.
//
// FP8 caches (OCP E4M3FN + per-row fp32 scale): codes become bf16 exactly when the tile is
// written to LDS; the K scale multiplies the logits of its key, the V scale multiplies P.
#pragma once

#include "mfma_tiles.h"

namespace hs2 {

constexpr int kRowWaves = 4;
constexpr int kRowListMax = 1280;   // list entries per workgroup (list mode)

// Registers of one tile in flight.
template <int D, int KV>
struct RowTile {
    static constexpr int NI = RawGeom<D, KV>::NI;
    u32x4_t k[NI];
    u32x4_t v[NI];
    int32_t kid;          // key id of row (lane & 31) of the tile; -1 = masked
    float ks, vs;         // fp8 scales of that row
};

// Issue the loads of one tile.  Every load is unconditional (rows are clamped into the valid
// range and masked keys are zeroed where the data is used), so the compiler counts outstanding
// loads exactly and keeps them in flight across the computation of the previous tile.
// LIST: `ids` holds the workgroup's key ids in LDS; otherwise (range mode) key = entry.
// Cache policy, measured on MI355X: in range mode (the full layer) K is loaded normally and V
// non-temporally, so V's lines do not displace K's from the memory-side cache before the score
// pass reads K again (decode128k: attention 103.5 -> 87 us, score pass 53.8 -> 47 us).  In list
// mode (the sparse layers) decode rows gather both non-temporally (cold 1152-row gathers of 256
// queries: 79 -> 49 us), while query chunks (REUSE), whose queries share window rows and
// often-chosen keys of one sequence, gather with cached loads (prefill_chunk: 380 -> 251 us).
template <int D, int KV, bool LIST, bool REUSE = false>
__device__ __forceinline__ void load_row_tile(RowTile<D, KV>& T, const AttnArgs& a, int64_t rowbase, int64_t L,
                                              int64_t e_lo, int64_t e_hi, int64_t tile_e, const int32_t* ids) {
    const int lane = threadIdx.x & 63;
    const int m = lane & 31;
    const int64_t e = tile_e + m;
    int64_t j;
    if (LIST) {
        const int64_t ec = e < e_hi ? e : e_hi - 1;
        j = ids[ec - e_lo];
        if (e >= e_hi || j < 0 || j >= L) j = -1;
    } else {
        j = e < e_hi ? e : -1;
    }
    T.kid = (int32_t)j;
    // a masked key reads the last key of the range (range mode) or row 0 (list mode)
    const int32_t jr = (int32_t)(j >= 0 ? j : (LIST ? 0 : e_hi - 1));
    auto src = [&](int R) { return rowbase + __shfl(jr, R); };
    load_raw_tile<D, KV, LIST && !REUSE>(T.k, a.k, src);
    load_raw_tile<D, KV, !(LIST && REUSE)>(T.v, a.v, src);
    if (KV == HS2_FP8_E4M3) {
        T.ks = a.k_scale[rowbase + jr];
        T.vs = a.v_scale[rowbase + jr];
    }
}

// Per-wave LDS of the row kernel: the K and V tiles and the fp8 scales of the tile's rows.
template <int D>
struct RowWaveLds {
    char k[LdsTile<D>::BYTES];
    char v[LdsTile<D>::BYTES];
    float ks[kTileRows];
    float vs[kTileRows];
};

// Stage a tile that has arrived in registers into the wave's LDS.  Returns the valid-row mask.
template <int D, int KV>
__device__ __forceinline__ uint32_t stage_row_tile(const RowTile<D, KV>& T, RowWaveLds<D>& W) {
    const int lane = threadIdx.x & 63;
    const uint32_t valid = (uint32_t)__ballot(T.kid >= 0);      // bit m: row m holds a key
    store_lds_tile<D, KV, false>(T.k, W.k, [](int) { return true; });
    store_lds_tile<D, KV, true>(T.v, W.v, [&](int R) { return (valid >> R) & 1u; });
    if (KV == HS2_FP8_E4M3 && lane < 32) { W.ks[lane] = T.ks; W.vs[lane] = T.vs; }
    return valid;
}

// Lanes l and l ^ 32 hold the two halves of a head's keys: v_permlane32_swap gives every lane
// both values without a trip through LDS.
__device__ __forceinline__ float half_max(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float half_sum(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// One 32-key tile: l_run is kept per lane half (the halves are added at the end).
template <int D, int KV>
__device__ __forceinline__ void row_tile_step(const RowWaveLds<D>& W, uint32_t valid, const char* qlds,
                                              f32x16_t* oacc, float& m_run, float& l_run, float sl2) {
    constexpr int KS = D / 16;
    constexpr int NB = D / 32;
    const int lane = threadIdx.x & 63;
    const int n = lane & 31, hb = lane >> 5;
    f32x16_t sacc = f32x16_t{};
#pragma unroll
    for (int s = 0; s < KS; ++s)
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row_operand<D>(W.k, n, hb * (D / 16) + s),
                                                       lds_row_operand<D>(qlds, n, hb * (D / 16) + s),
                                                       sacc, 0, 0, 0);
    // logits of keys m_i = 8(i/4) + 4hb + i%4 for head n
    float x[16];
    float ksc[16], vsc[16];
    if (KV == HS2_FP8_E4M3) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 a4 = *(const float4*)&W.ks[8 * g + 4 * hb];
            const float4 b4 = *(const float4*)&W.vs[8 * g + 4 * hb];
            ksc[4 * g] = a4.x; ksc[4 * g + 1] = a4.y; ksc[4 * g + 2] = a4.z; ksc[4 * g + 3] = a4.w;
            vsc[4 * g] = b4.x; vsc[4 * g + 1] = b4.y; vsc[4 * g + 2] = b4.z; vsc[4 * g + 3] = b4.w;
        }
    }
    float mt = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int m = 8 * (i >> 2) + 4 * hb + (i & 3);
        float sc = sl2;
        if (KV == HS2_FP8_E4M3) sc *= ksc[i];
        x[i] = ((valid >> m) & 1u) ? sacc[i] * sc : kNegInf;
        mt = fmaxf(mt, x[i]);
    }
    mt = half_max(mt);
    const float mn = fmaxf(m_run, mt);
    const float alpha = (mn == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - mn);
    // masked keys carry x = -inf and get weight exp2(-inf) = 0; while every key of a head has
    // been masked (mn = -inf) the reference point is 0, never -inf - (-inf)
    const float mref = (mn == kNegInf) ? 0.f : mn;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        x[i] = __builtin_amdgcn_exp2f(x[i] - mref);
        ps += x[i];
    }
    l_run = l_run * alpha + ps;
    m_run = mn;
    if (KV == HS2_FP8_E4M3) {
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] *= vsc[i];
    }
    // the running maximum rarely moves after the first tiles: rescale only when it did
    if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[blk][i] *= alpha;
    }
    bf16x8_t ph[2], pl[2];
    split_bf16x8(&x[0], ph[0], pl[0]);
    split_bf16x8(&x[8], ph[1], pl[1]);
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bf16x8_t av = lds_vt_operand<D>(W.v, blk, ks);
            oacc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, ph[ks], oacc[blk], 0, 0, 0);
            oacc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pl[ks], oacc[blk], 0, 0, 0);
        }
}

// ---- the attention kernel -------------------------------------------------------------------------
// Two workgroups (eight waves) per CU, so while one wave waits on LDS or MFMA results the other
// computes; each wave keeps its next tile in flight in registers.
// LDS of one workgroup of the row kernel.
template <int D>
struct RowLds {
    RowWaveLds<D> wl[kRowWaves];
    __attribute__((aligned(16))) char q[LdsTile<D>::BYTES];
    int32_t ids[kRowListMax];
    float ml[kRowWaves][32][2];
    float mlf[32][2];
};

// One workgroup's work: block row bx (row, or layer * R + row), key split `split`.  LIST: the
// keys are the index list a.list (sparse layers), otherwise the causal range (the full layer).
template <int D, int KV, bool LIST, bool REUSE = false>
__device__ __forceinline__ void attn_rows_body(const AttnArgs& a, int bx, int split, RowLds<D>& S) {
    constexpr int NW = kRowWaves;
    constexpr int NT = NW * 64;
    constexpr int NB = D / 32;

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = lane & 31, hb = lane >> 5;
    int r = bx;
    const void* qsrc = a.q;
    float* odst = a.o;
    float* part = a.part;
    float* part_ml = a.part_ml;
    if (a.nlayer > 1) {
        const int R = a.B * a.Tq, layer = r / R;
        r -= layer * R;
        qsrc = a.ql[layer];
        odst = a.ol[layer];
        if (part) {
            part += layer * a.part_lstride;
            part_ml += layer * a.ml_lstride;
        }
    }
    const int b = r / a.Tq;
    const int H = a.H;
    const int64_t L = seq_len(a.kv_len, b, a.Nmax);
    int64_t e0 = (int64_t)split * a.chunk, e1;
    if (LIST) {
        e1 = e0 + a.chunk < a.S ? e0 + a.chunk : a.S;
        if (e1 - e0 > kRowListMax) e1 = e0 + kRowListMax;   // the host never plans more
    } else {
        const int64_t t = row_pos(a.q_pos, a.kv_len, r, a.Tq, a.Nmax);
        e1 = e0 + a.chunk < t + 1 ? e0 + a.chunk : t + 1;
    }
    const int64_t ntiles = e1 > e0 ? (e1 - e0 + 31) / 32 : 0;
    // this row's selection workspace is cleared here, before the score pass accumulates into it
    if (a.zero_hist && split == 0) {
        for (int x = threadIdx.x; x < kHistBins; x += NT) a.zero_hist[(int64_t)r * kHistBins + x] = 0;
        if (threadIdx.x < 4) a.zero_cnt[(int64_t)r * 4 + threadIdx.x] = 0;
    }
    // Prologue: Q (heads padded to 32 with zeros) becomes an LDS tile, the Q^T operand of every
    // MFMA step, and the workgroup's list entries go to LDS.  Every load of the prologue is issued
    // before the first one is used, so it costs one memory round trip instead of one per loop pass.
    constexpr int CPR = LdsTile<D>::CPR;
    constexpr int QX = (32 * CPR + NT - 1) / NT;
    constexpr int IX = LIST ? (kRowListMax + NT - 1) / NT : 0;
    const int32_t* ids = nullptr;
    {
        const u32x4_t* qp = (const u32x4_t*)((const uint16_t*)qsrc + (int64_t)r * H * D);
        u32x4_t qv[QX];
#pragma unroll
        for (int x = 0; x < QX; ++x) {
            const int f = threadIdx.x + x * NT, h = f / CPR, c = f % CPR;
            qv[x] = u32x4_t{0, 0, 0, 0};
            if (f < 32 * CPR && h < H) qv[x] = qp[h * CPR + c];
        }
        int32_t iv[IX > 0 ? IX : 1];
#pragma unroll
        for (int x = 0; x < IX; ++x) {
            const int64_t e = threadIdx.x + (int64_t)x * NT;
            iv[x] = -1;
            if (e < e1 - e0) iv[x] = a.list[(int64_t)r * a.S + e0 + e];
        }
#pragma unroll
        for (int x = 0; x < QX; ++x) {
            const int f = threadIdx.x + x * NT;
            if (f < 32 * CPR) *(u32x4_t*)(S.q + LdsTile<D>::off(f / CPR, f % CPR)) = qv[x];
        }
#pragma unroll
        for (int x = 0; x < IX; ++x) {
            const int64_t e = threadIdx.x + (int64_t)x * NT;
            if (e < e1 - e0) S.ids[e] = iv[x];
        }
        if (LIST) ids = S.ids;
    }
    __syncthreads();
    RowWaveLds<D>& W = S.wl[w];
    f32x16_t oacc[NB];
#pragma unroll
    for (int x = 0; x < NB; ++x) oacc[x] = f32x16_t{};
    float m_run = kNegInf, l_run = 0.f;
    const float sl2 = a.scale_log2;
    const int64_t rowbase = (int64_t)b * a.Nmax;

    // one tile in registers in flight while the previous one is computed from LDS; the loop
    // loads unconditionally and the wave's last tile is peeled off, so no load is issued past it
    RowTile<D, KV> T;
    const int64_t ntw = ntiles > w ? (ntiles - w + NW - 1) / NW : 0;   // tiles of this wave
    if (ntw > 0) {
        auto tile_e = [&](int64_t it) { return e0 + 32 * (w + (int64_t)NW * it); };
        load_row_tile<D, KV, LIST, REUSE>(T, a, rowbase, L, e0, e1, tile_e(0), ids);
        for (int64_t it = 0; it + 1 < ntw; ++it) {
            const uint32_t valid = stage_row_tile<D, KV>(T, W);
            load_row_tile<D, KV, LIST, REUSE>(T, a, rowbase, L, e0, e1, tile_e(it + 1), ids);
            wave_lds_fence();
            row_tile_step<D, KV>(W, valid, S.q, oacc, m_run, l_run, sl2);
            wave_lds_fence();
        }
        const uint32_t valid = stage_row_tile<D, KV>(T, W);
        wave_lds_fence();
        row_tile_step<D, KV>(W, valid, S.q, oacc, m_run, l_run, sl2);
        wave_lds_fence();
    }

    l_run = half_sum(l_run);

    // ---- merge the waves of the workgroup ----
    // every lane combines the (m, l) of its head n over the waves and keeps its own wave's scale
    if (lane < 32) { S.ml[w][n][0] = m_run; S.ml[w][n][1] = l_run; }
    __syncthreads();
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, S.ml[ww][n][0]);
    float Lsum = 0.f, myscale = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
        const float mw = S.ml[ww][n][0];
        const float sc = mw == kNegInf ? 0.f : exp2f(mw - M);
        Lsum += S.ml[ww][n][1] * sc;
        if (ww == w) myscale = sc;
    }
    if (w == 0 && lane < 32) { S.mlf[n][0] = M; S.mlf[n][1] = Lsum; }
    // each wave stores its scaled O^T in its own (now idle) tile space as float4s of four
    // consecutive dv: float4 q = dv / 4 of head n sits at n * QN + (q ^ (n mod QN)), which keeps
    // these stores and the cross-wave loads below free of bank conflicts
    constexpr int QN = D / 4;
    {
        float4* ob = (float4*)&S.wl[w];
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int q = 8 * blk + 2 * g + hb;          // dv = 32 blk + 8 g + 4 hb + j
                ob[n * QN + (q ^ (n & (QN - 1)))] =
                    make_float4(oacc[blk][4 * g] * myscale, oacc[blk][4 * g + 1] * myscale,
                                oacc[blk][4 * g + 2] * myscale, oacc[blk][4 * g + 3] * myscale);
            }
    }
    __syncthreads();
    const bool o_vec = ((uintptr_t)odst & 15) == 0;
    for (int f = threadIdx.x; f < H * QN; f += NT) {
        const int h = f / QN, q = f % QN;
        const int slot = h * QN + (q ^ (h & (QN - 1)));
        float4 sum = ((const float4*)&S.wl[0])[slot];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) {
            const float4 v = ((const float4*)&S.wl[ww])[slot];
            sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
        }
        if (part) {
            *(float4*)(part + (((int64_t)r * a.nsplit + split) * H + h) * D + 4 * q) = sum;
        } else {
            const float Lh = S.mlf[h][1];
            const float inv = Lh > 0.f ? 1.f / Lh : 0.f;
            float* op = odst + ((int64_t)r * H + h) * D + 4 * q;
            if (o_vec) {
                *(float4*)op = make_float4(sum.x * inv, sum.y * inv, sum.z * inv, sum.w * inv);
            } else {
                op[0] = sum.x * inv; op[1] = sum.y * inv; op[2] = sum.z * inv; op[3] = sum.w * inv;
            }
        }
    }
    if (threadIdx.x < H) {
        const float Mh = S.mlf[threadIdx.x][0], Lh = S.mlf[threadIdx.x][1];
        if (part)
            *(float2*)(part_ml + (((int64_t)r * a.nsplit + split) * H + threadIdx.x) * 2) = make_float2(Mh, Lh);
        else if (a.lse)
            a.lse[(int64_t)r * H + threadIdx.x] = Lh > 0.f ? Mh + log2f(Lh) : kNegInf;
    }
}

}  // namespace hs2
