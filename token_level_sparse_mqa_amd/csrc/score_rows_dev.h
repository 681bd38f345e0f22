// Selection-score pass of the decode (row) path on MFMA.
//
// Score (the selection score fixed for this library; see include/hs2.h): for query row t and
// candidate key j in [0, t - window], score(j) = sum over heads h of the full layer's softmax
// probability 2^(x_h(j) - lse_h), x in base 2, lse_h the row's base-2 log-sum-exp from the
// attention pass.  The pass also accumulates the row histogram of the scores' top radix digit
// for the selection kernels.
#pragma once

#include "mfma_tiles.h"

namespace hs2 {

constexpr int kScoreWaves = 4;

// ---- score pass --------------------------------------------------------------------------------
// score(j) = sum_h 2^(x_h(j) - lse_h) for candidates j in [0, t - window]; S[head][key] = Q . K^T
// so that every lane owns one key and sums its 16 heads, plus the partner lane's 16.
//
// K needs no LDS here: the B operand of lane (key n, half hb) at k-step s is 8 consecutive d
// of key n, so each lane loads its operands straight from the cache row with 16-byte loads.
// The d order inside the product is free as long as Q uses the same one; it is chosen so that
// one load instruction covers 32 consecutive bytes of each of its 32 rows (one cache line per
// row):  bf16: k-step s <-> d in [16s + 8hb, +8);  FP8: lane half hb holds d in [hb*D/2, +D/2),
// k-step s <-> d in [hb*D/2 + 8s, +8).  NBUF tiles stay in flight per wave.
struct ScoreLds {
    uint32_t hist[kHistBins];
};

// One workgroup of 256 threads: row bx, split number by (splits run last-to-first, so the
// workgroup of by = 0 takes the last split).
template <int D, int KV>
__device__ __forceinline__ void score_rows_body(const ScoreArgs& a, int bx, int by, ScoreLds& S) {
    constexpr int KS = D / 16;
    constexpr int ESZ = KV == HS2_FP8_E4M3 ? 1 : 2;
    constexpr int RB = D * ESZ;                  // bytes per cache row
    constexpr int NL = RB / 32;                  // 16-byte loads per lane per tile (half a row)
    constexpr int NBUF = KV == HS2_FP8_E4M3 ? 6 : 4;
    uint32_t (&hist)[kHistBins] = S.hist;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = lane & 31, hb = lane >> 5;
    // splits run last-to-first: the attention pass streamed the cache first-to-last, so the
    // keys it read last are the likeliest to still sit in the memory-side cache
    const int r = bx, split = a.nsplit - 1 - by;
    const int b = r / a.Tq;
    const int H = a.H;
    const int64_t t = row_pos(a.q_pos, a.kv_len, r, a.Tq, a.Nmax);
    const int64_t C = cand_count(t, a.window);
    const int64_t e0 = (int64_t)split * a.chunk;
    const int64_t e1 = e0 + a.chunk < C ? e0 + a.chunk : C;
    if (e0 >= e1) return;
    const int64_t ntiles = (e1 - e0 + 31) / 32;
    if (a.rowhist)
        for (int x = threadIdx.x; x < kHistBins; x += 256) hist[x] = 0;

    // Q rows and the normalisers are loaded unconditionally (clamped head, zeroed by select), so
    // all of them are in flight together instead of one exec-masked load at a time
    bf16x8_t qop[KS];
    {
        const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)r * H + (n < H ? n : H - 1)) * D;
        const uint32_t keep = n < H ? 0xffffffffu : 0u;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int d0 = KV == HS2_FP8_E4M3 ? hb * (D / 2) + 8 * s : 16 * s + 8 * hb;
            u32x4_t v = *(const u32x4_t*)(qrow + d0);
            v[0] &= keep; v[1] &= keep; v[2] &= keep; v[3] &= keep;
            qop[s] = __builtin_bit_cast(bf16x8_t, v);
        }
    }
    // negative base-2 log normaliser of the 16 heads this lane sums: heads 8(i/4) + 4hb + i%4
    float nlse[16];
    {
        const float* lr = a.lse + (int64_t)r * H;
        float raw[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int h = 8 * (i >> 2) + 4 * hb + (i & 3);
            raw[i] = lr[h < H ? h : H - 1];
        }
        // padded heads get -inf through arithmetic on the loaded value (a select would let the
        // compiler turn the load back into a masked one)
#pragma unroll
        for (int i = 0; i < 16; ++i) nlse[i] = -raw[i] - (8 * (i >> 2) + 4 * hb + (i & 3) < H ? 0.f : kPosInf);
    }
    if (a.rowhist) __syncthreads();

    u32x4_t kb[NBUF][NL];
    float ksb[NBUF];
    const int64_t ntw = ntiles > w ? (ntiles - w + kScoreWaves - 1) / kScoreWaves : 0;
    // bf16: load x of lane (n, hb) is row bytes [32x + 16hb, +16); FP8: [hb*RB/2 + 16x, +16)
    const char* kbase = (const char*)a.k + (int64_t)b * a.Nmax * RB + (KV == HS2_FP8_E4M3 ? hb * (RB / 2) : 16 * hb);
    constexpr int LSTRIDE = KV == HS2_FP8_E4M3 ? 16 : 32;
    const float* ksbase = KV == HS2_FP8_E4M3 ? a.k_scale + (int64_t)b * a.Nmax : nullptr;
    // unconditional loads (keys clamped into the range, prefetches past the end re-load the
    // wave's last tile) keep the compiler's load counting exact
    auto load = [&](u32x4_t* kr, float& ks, int64_t it) {
        const int64_t tl = w + (int64_t)kScoreWaves * (it < ntw ? it : ntw - 1);
        const int64_t j = e0 + 32 * tl + n < e1 ? e0 + 32 * tl + n : e1 - 1;
        const char* p = kbase + j * RB;
#pragma unroll
        for (int x = 0; x < NL; ++x) kr[x] = ld16<false>(p + LSTRIDE * x);
        if (KV == HS2_FP8_E4M3) ks = ksbase[j];
    };
    auto kop = [&](const u32x4_t* kr, int s) -> bf16x8_t {
        if (KV == HS2_FP8_E4M3) {
            const u32x4_t c = kr[s >> 1];
            const u32x2_t lo = fp8x4_to_bf16x4(c[2 * (s & 1)]), hi = fp8x4_to_bf16x4(c[2 * (s & 1) + 1]);
            u32x4_t o;
            o[0] = lo[0]; o[1] = lo[1]; o[2] = hi[0]; o[3] = hi[1];
            return __builtin_bit_cast(bf16x8_t, o);
        }
        return __builtin_bit_cast(bf16x8_t, kr[s]);
    };
    float* srow = a.scores + (int64_t)r * a.cstride;
    if (ntw > 0) {
#pragma unroll
        for (int u = 0; u < NBUF - 1; ++u) load(kb[u], ksb[u], u);
        for (int64_t base = 0; base < ntw; base += NBUF) {
#pragma unroll
            for (int u = 0; u < NBUF; ++u) {
                const int64_t it = base + u;
                load(kb[(u + NBUF - 1) % NBUF], ksb[(u + NBUF - 1) % NBUF], it + NBUF - 1);
                if (it < ntw) {
                    const int64_t tile = w + (int64_t)kScoreWaves * it;
                    f32x16_t sacc = f32x16_t{};
#pragma unroll
                    for (int s = 0; s < KS; ++s)
                        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qop[s], kop(kb[u], s), sacc, 0, 0, 0);
                    float sc = a.scale_log2;
                    if (KV == HS2_FP8_E4M3) sc *= ksb[u];
                    float acc = 0.f;
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc += __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], sc, nlse[i]));
                    // The partner lane holds the other 16 heads. An LDS permute here, not the 32-lane
                    // swap: this loop is bound by vector issue, and the permute's latency hides behind it.
                    acc += __shfl_xor(acc, 32);
                    const int64_t j = e0 + 32 * tile + n;
                    if (hb == 0 && j < e1) {
                        srow[j] = acc;
                        if (a.rowhist) atomicAdd(&hist[__float_as_uint(acc) >> 21], 1u);
                    }
                }
            }
        }
    }
    if (a.rowhist) {
        __syncthreads();
        for (int x = threadIdx.x; x < kHistBins; x += 256)
            if (hist[x]) atomicAdd(&a.rowhist[(int64_t)r * kHistBins + x], hist[x]);
    }
}

}  // namespace hs2
