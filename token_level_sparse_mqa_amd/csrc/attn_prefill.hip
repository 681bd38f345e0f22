// MFMA kernels for query chunks (prefill): the full-attention pass and the score pass.
//
// A chunk of new tokens attends causally over the cache (agentik-os article, section 1: a long
// observation is prefilled into a growing context).  MQA lets the eight query tokens of a
// workgroup share every K/V tile: the tile is read from memory once into LDS and all eight
// waves (one query token each, its 32 heads as the MFMA N dimension) multiply against it.
//
// Pass 1 per wave and 32-key tile:
//   S^T = K_tile . Q^T (bf16 MFMA), causal mask key <= t, online softmax in base 2,
//   O^T += V^T . P^T with V staged in LDS as fp16 and P rounded to fp16 (fp16 MFMA).
// Pass 2 (score) per wave and tile:
//   S = Q . K_tile^T, score(j) = sum_h 2^(x_h(j) - lse_h), a per-row radix histogram in LDS.
//
// Workgroup tiles are double-buffered in LDS; the cooperative global loads of the next tiles
// are kept in flight in registers (unconditional, clamped loads) while a tile is computed.
#include "mfma_tiles.h"

namespace hs2 {

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;

constexpr int kPfWaves = 8;                  // query tokens (waves) per workgroup
constexpr int kPfThreads = kPfWaves * 64;

// Geometry of the cooperative (workgroup-wide) loads of one tile in storage format.
template <int D, int KV>
struct PfGeom {
    using G = RawGeom<D, KV>;
    static constexpr int CHUNKS = kTileRows * G::CPR;                    // 16-byte chunks per tile
    static constexpr int NX = (CHUNKS + kPfThreads - 1) / kPfThreads;    // loads per thread
};

// Per-thread part of the cooperative tile loads: load x of a thread reads 16-byte chunk c of tile
// row R, at byte offset (k0 + R) * RB + 16 c from the sequence's first cache row.  Offsets are
// 32-bit (the host keeps Nmax * row bytes below 2^31).
template <int D, int KV>
struct PfLoader {
    using G = RawGeom<D, KV>;
    using P = PfGeom<D, KV>;
    uint32_t off[P::NX];      // R * RB + 16 c
    int R[P::NX];
    __device__ __forceinline__ PfLoader() {
#pragma unroll
        for (int x = 0; x < P::NX; ++x) {
            int q = threadIdx.x + x * kPfThreads;
            q = q < P::CHUNKS ? q : P::CHUNKS - 1;
            R[x] = q / G::CPR;
            off[x] = (uint32_t)(R[x] * G::RB + 16 * (q % G::CPR));
        }
    }
    // rows k0 .. k0+31; rows at or past khi read row khi - 1 instead
    __device__ __forceinline__ void load(u32x4_t* raw, const char* seq, int64_t k0, int64_t khi) const {
        if (k0 + kTileRows <= khi) {
            const uint32_t base = (uint32_t)k0 * G::RB;
#pragma unroll
            for (int x = 0; x < P::NX; ++x) raw[x] = *(const u32x4_t*)(seq + (base + off[x]));
        } else {
#pragma unroll
            for (int x = 0; x < P::NX; ++x) {
                const int64_t key = k0 + R[x] < khi ? k0 + R[x] : khi - 1;
                raw[x] = *(const u32x4_t*)(seq + ((uint32_t)key * G::RB + (off[x] - (uint32_t)R[x] * G::RB)));
            }
        }
    }
};

// bf16 LDS tile from raw K (FP8 codes converted exactly).
template <int D, int KV>
__device__ __forceinline__ void pf_store_k(const u32x4_t* raw, char* lds) {
    using G = RawGeom<D, KV>;
    using P = PfGeom<D, KV>;
    using T = LdsTile<D>;
#pragma unroll
    for (int x = 0; x < P::NX; ++x) {
        const int q = threadIdx.x + x * kPfThreads;
        if (q >= P::CHUNKS) continue;
        const int R = q / G::CPR, c = q % G::CPR;
        if (KV == HS2_FP8_E4M3) {
            u32x4_t lo, hi;
            const u32x2_t a = fp8x4_to_bf16x4(raw[x][0]), b = fp8x4_to_bf16x4(raw[x][1]);
            const u32x2_t cc = fp8x4_to_bf16x4(raw[x][2]), d = fp8x4_to_bf16x4(raw[x][3]);
            lo[0] = a[0]; lo[1] = a[1]; lo[2] = b[0]; lo[3] = b[1];
            hi[0] = cc[0]; hi[1] = cc[1]; hi[2] = d[0]; hi[3] = d[1];
            *(u32x4_t*)(lds + T::off(R, 2 * c)) = lo;
            *(u32x4_t*)(lds + T::off(R, 2 * c + 1)) = hi;
        } else {
            *(u32x4_t*)(lds + T::off(R, c)) = raw[x];
        }
    }
}

__device__ __forceinline__ uint32_t f16x2_bits(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// fp16 LDS tile from raw V.  bf16 -> fp16 is exact for |v| in [2^-14, 65504]; smaller values
// keep an absolute error below 2^-25, larger ones saturate.  FP8 codes convert exactly.
template <int D, int KV>
__device__ __forceinline__ void pf_store_v(const u32x4_t* raw, char* lds) {
    using G = RawGeom<D, KV>;
    using P = PfGeom<D, KV>;
    using T = LdsTile<D>;
#pragma unroll
    for (int x = 0; x < P::NX; ++x) {
        const int q = threadIdx.x + x * kPfThreads;
        if (q >= P::CHUNKS) continue;
        const int R = q / G::CPR, c = q % G::CPR;
        if (KV == HS2_FP8_E4M3) {
            u32x4_t lo, hi;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const f32x2_t a = fp8x2_to_f32<false>(raw[x][w]), b = fp8x2_to_f32<true>(raw[x][w]);
                const uint32_t p0 = f16x2_bits(a[0], a[1]), p1 = f16x2_bits(b[0], b[1]);
                if (w < 2) { lo[2 * w] = p0; lo[2 * w + 1] = p1; } else { hi[2 * w - 4] = p0; hi[2 * w - 3] = p1; }
            }
            *(u32x4_t*)(lds + T::voff(R, 2 * c)) = lo;
            *(u32x4_t*)(lds + T::voff(R, 2 * c + 1)) = hi;
        } else {
            u32x4_t o;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t u = raw[x][w];
                o[w] = f16x2_bits(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
            }
            *(u32x4_t*)(lds + T::voff(R, c)) = o;
        }
    }
}

template <int D>
__device__ __forceinline__ f16x8_t lds_vt_operand_f16(const char* lds, int blk, int ks) {
    return __builtin_bit_cast(f16x8_t, lds_vt_operand<D>(lds, blk, ks));
}

// Positions of the workgroup's query rows; returns the largest one (or -1).
__device__ __forceinline__ int64_t pf_rows(const int32_t* q_pos, const int32_t* kv_len, int Tq, int64_t Nmax,
                                           int b, int i0, int64_t* t_s) {
    if (threadIdx.x < kPfWaves) {
        const int i = i0 + threadIdx.x;
        t_s[threadIdx.x] = i < Tq ? row_pos(q_pos, kv_len, b * Tq + i, Tq, Nmax) : -1;
    }
    __syncthreads();
    int64_t tmax = -1;
#pragma unroll
    for (int w = 0; w < kPfWaves; ++w) tmax = t_s[w] > tmax ? t_s[w] : tmax;
    return tmax;
}

// ---- pass 1 -------------------------------------------------------------------------------------
// Lanes l and l ^ 32 hold the two halves of a head's keys: v_permlane32_swap gives every lane
// both values without a trip through LDS.
__device__ __forceinline__ float pf_half_max(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float pf_half_sum(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// One barrier per stage of SUB 32-key sub-tiles: each wave multiplies both sub-tiles, then runs
// one online-softmax step over the 16 * SUB logits a lane holds for its head, so the barrier,
// the maximum exchange and the rescale test are paid once per 64 keys.
template <int D, int KV>
__global__ __launch_bounds__(kPfThreads, 1) void attn_prefill_kernel(AttnArgs a) {
    constexpr int KS = D / 16, NB = D / 32;
    constexpr int NX = PfGeom<D, KV>::NX;
    constexpr int SUB = 2;                       // 32-key sub-tiles per stage
    constexpr int SK = SUB * kTileRows;          // keys per stage
    constexpr int NST = 2;                       // stages in flight in registers
    __shared__ __attribute__((aligned(16))) char kt[2][SUB][LdsTile<D>::BYTES];
    __shared__ __attribute__((aligned(16))) char vt[2][SUB][LdsTile<D>::BYTES];
    __shared__ float ks_s[2][SUB][kTileRows], vs_s[2][SUB][kTileRows];
    __shared__ int64_t t_s[kPfWaves];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = lane & 31, hb = lane >> 5;
    const int nqt = (a.Tq + kPfWaves - 1) / kPfWaves;
    const int b = blockIdx.x / nqt, i0 = (blockIdx.x % nqt) * kPfWaves;
    const int H = a.H;
    const int64_t tmax = pf_rows(a.q_pos, a.kv_len, a.Tq, a.Nmax, b, i0, t_s);
    const int64_t t = t_s[w];
    const int r = b * a.Tq + (i0 + w < a.Tq ? i0 + w : a.Tq - 1);
    const int64_t nstages = (tmax + 1 + SK - 1) / SK;
    const int64_t rowbase = (int64_t)b * a.Nmax;
    // the selection counters of these rows are cleared here (the score pass writes the whole
    // radix histogram of each row itself)
    if (a.zero_cnt && threadIdx.x < 4 * kPfWaves && i0 + (int)threadIdx.x / 4 < a.Tq)
        a.zero_cnt[((int64_t)b * a.Tq + i0) * 4 + threadIdx.x] = 0;

    bf16x8_t qop[KS];
    {
        const u32x4_t* qp = (const u32x4_t*)((const uint16_t*)a.q + ((int64_t)r * H + (n < H ? n : 0)) * D + hb * (D / 2));
#pragma unroll
        for (int s = 0; s < KS; ++s) qop[s] = n < H ? __builtin_bit_cast(bf16x8_t, qp[s]) : bf16x8_t{};
    }
    f32x16_t oacc[NB];
#pragma unroll
    for (int x = 0; x < NB; ++x) oacc[x] = f32x16_t{};
    float m_run = kNegInf, l_run = 0.f;          // l_run per lane half
    const float sl2 = a.scale_log2;

    if (nstages > 0) {
        const int64_t khi = tmax + 1;
        const char* kseq = (const char*)a.k + rowbase * RawGeom<D, KV>::RB;
        const char* vseq = (const char*)a.v + rowbase * RawGeom<D, KV>::RB;
        const PfLoader<D, KV> ld;
        u32x4_t rk[NST][SUB][NX], rv[NST][SUB][NX];
        float rks[NST][SUB], rvs[NST][SUB];
        auto load = [&](int st, int64_t stage) {
            const int64_t sg = stage < nstages ? stage : nstages - 1;
#pragma unroll
            for (int sub = 0; sub < SUB; ++sub) {
                const int64_t k0 = sg * SK + sub * kTileRows;
                ld.load(rk[st][sub], kseq, k0, khi);
                ld.load(rv[st][sub], vseq, k0, khi);
                if (KV == HS2_FP8_E4M3) {
                    const int64_t key = k0 + (threadIdx.x & 31);
                    const int64_t kc = key < khi ? key : khi - 1;
                    rks[st][sub] = a.k_scale[rowbase + kc];
                    rvs[st][sub] = a.v_scale[rowbase + kc];
                }
            }
        };
        auto store = [&](int st, int buf) {
#pragma unroll
            for (int sub = 0; sub < SUB; ++sub) {
                pf_store_k<D, KV>(rk[st][sub], kt[buf][sub]);
                pf_store_v<D, KV>(rv[st][sub], vt[buf][sub]);
                if (KV == HS2_FP8_E4M3 && threadIdx.x < kTileRows) {
                    ks_s[buf][sub][threadIdx.x] = rks[st][sub];
                    vs_s[buf][sub][threadIdx.x] = rvs[st][sub];
                }
            }
        };
#pragma unroll
        for (int u = 0; u < NST; ++u) load(u, u);
        store(0, 0);
        __syncthreads();
        for (int64_t base = 0; base < nstages; base += NST) {
#pragma unroll
            for (int u = 0; u < NST; ++u) {
                const int64_t stage = base + u;
                if (stage >= nstages) break;
                const int buf = (int)(stage & 1);
                const int64_t k0 = stage * SK;
                if (k0 <= t) {
                    f32x16_t sacc[SUB];
#pragma unroll
                    for (int sub = 0; sub < SUB; ++sub) {
                        sacc[sub] = f32x16_t{};
#pragma unroll
                        for (int s = 0; s < KS; ++s)
                            sacc[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                lds_row_operand<D>(kt[buf][sub], n, hb * (D / 16) + s), qop[s], sacc[sub], 0, 0, 0);
                    }
                    // logits x = s * sc (sc > 0); keys past t are masked in the stage holding t
                    float x[16 * SUB];
#pragma unroll
                    for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int kr = 8 * (i >> 2) + 4 * hb + (i & 3);    // key row in the sub-tile
                            x[16 * sub + i] = KV == HS2_FP8_E4M3 ? sacc[sub][i] * (sl2 * ks_s[buf][sub][kr]) : sacc[sub][i];
                        }
                    if (k0 + SK - 1 > t) {
                        const int lim = (int)(t - k0);
#pragma unroll
                        for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
                            for (int i = 0; i < 16; ++i)
                                if (kTileRows * sub + 8 * (i >> 2) + 4 * hb + (i & 3) > lim) x[16 * sub + i] = kNegInf;
                    }
                    float mt = x[0];
#pragma unroll
                    for (int i = 1; i < 16 * SUB; ++i) mt = fmaxf(mt, x[i]);
                    mt = pf_half_max(mt);
                    // bf16 path: x is still unscaled, scale the maximum (sc > 0 keeps the order)
                    const float scl = KV == HS2_FP8_E4M3 ? 1.f : sl2;
                    const float mn = fmaxf(m_run, mt * scl);
                    const float alpha = (mn == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - mn);
                    const float mref = (mn == kNegInf) ? 0.f : mn;
                    float ps = 0.f;
#pragma unroll
                    for (int i = 0; i < 16 * SUB; ++i) {
                        x[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], scl, -mref));
                        ps += x[i];
                    }
                    l_run = l_run * alpha + ps;
                    m_run = mn;
                    if (KV == HS2_FP8_E4M3) {
#pragma unroll
                        for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
                            for (int i = 0; i < 16; ++i) x[16 * sub + i] *= vs_s[buf][sub][8 * (i >> 2) + 4 * hb + (i & 3)];
                    }
                    if (__ballot(alpha != 1.f)) {
#pragma unroll
                        for (int blk = 0; blk < NB; ++blk)
#pragma unroll
                            for (int i = 0; i < 16; ++i) oacc[blk][i] *= alpha;
                    }
                    f16x8_t p[SUB][2];
#pragma unroll
                    for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            p[sub][0][e] = (_Float16)x[16 * sub + e];
                            p[sub][1][e] = (_Float16)x[16 * sub + 8 + e];
                        }
#pragma unroll
                    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
                        for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
                            for (int ks = 0; ks < 2; ++ks)
                                oacc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                    lds_vt_operand_f16<D>(vt[buf][sub], blk, ks), p[sub][ks], oacc[blk], 0, 0, 0);
                }
                // stage + 1 (registers (u+1) % NST) into the other buffer, refill registers u
                if (stage + 1 < nstages) store((u + 1) % NST, buf ^ 1);
                load(u, stage + NST);
                __syncthreads();
            }
        }
    }
    l_run = pf_half_sum(l_run);

    // ---- finish: this workgroup saw every key of its rows ----
    if (i0 + w < a.Tq) {
        const float linv = l_run > 0.f ? 1.f / l_run : 0.f;
        float* po = a.o + ((int64_t)r * H) * D;
        if (n < H) {
#pragma unroll
            for (int blk = 0; blk < NB; ++blk)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int dv = blk * 32 + 8 * g + 4 * hb;
                    float4 v4;
                    v4.x = oacc[blk][4 * g] * linv; v4.y = oacc[blk][4 * g + 1] * linv;
                    v4.z = oacc[blk][4 * g + 2] * linv; v4.w = oacc[blk][4 * g + 3] * linv;
                    *(float4*)(po + n * D + dv) = v4;
                }
            if (hb == 0 && a.lse) a.lse[(int64_t)r * H + n] = l_run > 0.f ? m_run + log2f(l_run) : kNegInf;
        }
    }
}

// ---- pass 2: selection scores ---------------------------------------------------------------------
template <int D, int KV>
__global__ __launch_bounds__(kPfThreads, 1) void score_prefill_kernel(ScoreArgs a) {
    constexpr int KS = D / 16;
    constexpr int NX = PfGeom<D, KV>::NX;
    constexpr int NST = 4;
    __shared__ __attribute__((aligned(16))) char kt[2][LdsTile<D>::BYTES];
    __shared__ float ks_s[2][kTileRows];
    __shared__ uint32_t hist[kPfWaves][kHistBins];
    __shared__ int64_t t_s[kPfWaves];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = lane & 31, hb = lane >> 5;
    const int nqt = (a.Tq + kPfWaves - 1) / kPfWaves;
    const int b = blockIdx.x / nqt, i0 = (blockIdx.x % nqt) * kPfWaves;
    const int H = a.H;
    const int64_t tmax = pf_rows(a.q_pos, a.kv_len, a.Tq, a.Nmax, b, i0, t_s);
    const int64_t t = t_s[w];
    const bool live = i0 + w < a.Tq;
    const int r = b * a.Tq + (live ? i0 + w : a.Tq - 1);
    const int64_t C = cand_count(t, a.window);
    const int64_t Cmax = cand_count(tmax, a.window);
    const int64_t ntiles = (Cmax + kTileRows - 1) / kTileRows;
    const int64_t rowbase = (int64_t)b * a.Nmax;
    for (int x = threadIdx.x; x < kPfWaves * kHistBins; x += kPfThreads) (&hist[0][0])[x] = 0;

    bf16x8_t qop[KS];
    {
        const u32x4_t* qp = (const u32x4_t*)((const uint16_t*)a.q + ((int64_t)r * H + (n < H ? n : 0)) * D + hb * (D / 2));
#pragma unroll
        for (int s = 0; s < KS; ++s) qop[s] = n < H ? __builtin_bit_cast(bf16x8_t, qp[s]) : bf16x8_t{};
    }
    float nlse[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int h = 8 * (i >> 2) + 4 * hb + (i & 3);
        nlse[i] = (h < H && C > 0) ? -a.lse[(int64_t)r * H + h] : kNegInf;
    }
    float* srow = a.scores + (int64_t)r * a.cstride;

    if (ntiles > 0) {
        const char* kseq = (const char*)a.k + rowbase * RawGeom<D, KV>::RB;
        const PfLoader<D, KV> ld;
        u32x4_t rk[NST][NX];
        float rks[NST];
        auto load = [&](int st, int64_t tile) {
            const int64_t tl = tile < ntiles ? tile : ntiles - 1;
            ld.load(rk[st], kseq, tl * kTileRows, Cmax);
            if (KV == HS2_FP8_E4M3) {
                const int64_t key = tl * kTileRows + (threadIdx.x & 31);
                rks[st] = a.k_scale[rowbase + (key < Cmax ? key : Cmax - 1)];
            }
        };
        auto store = [&](int st, int buf) {
            pf_store_k<D, KV>(rk[st], kt[buf]);
            if (KV == HS2_FP8_E4M3 && threadIdx.x < kTileRows) ks_s[buf][threadIdx.x] = rks[st];
        };
#pragma unroll
        for (int u = 0; u < NST; ++u) load(u, u);
        store(0, 0);
        __syncthreads();
        for (int64_t base = 0; base < ntiles; base += NST) {
#pragma unroll
            for (int u = 0; u < NST; ++u) {
                const int64_t tile = base + u;
                if (tile >= ntiles) break;
                const int buf = (int)(tile & 1);
                const int64_t k0 = tile * kTileRows;
                if (k0 < C) {
                    f32x16_t sacc = f32x16_t{};
#pragma unroll
                    for (int s = 0; s < KS; ++s)
                        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qop[s], lds_row_operand<D>(kt[buf], n, hb * (D / 16) + s),
                                                                       sacc, 0, 0, 0);
                    float sc = a.scale_log2;
                    if (KV == HS2_FP8_E4M3) sc *= ks_s[buf][n];
                    float acc = 0.f;
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc += __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], sc, nlse[i]));
                    acc += __shfl_xor(acc, 32);
                    const int64_t j = k0 + n;
                    if (hb == 0 && j < C) {
                        srow[j] = acc;
                        atomicAdd(&hist[w][__float_as_uint(acc) >> 21], 1u);
                    }
                }
                if (tile + 1 < ntiles) store((u + 1) % NST, buf ^ 1);
                load(u, tile + NST);
                __syncthreads();
            }
        }
    }
    // this workgroup owns its rows' histograms entirely
    __syncthreads();
    if (a.rowhist) {
        for (int x = threadIdx.x; x < kPfWaves * kHistBins; x += kPfThreads) {
            const int ww = x / kHistBins;
            if (i0 + ww < a.Tq) a.rowhist[((int64_t)b * a.Tq + i0 + ww) * kHistBins + (x % kHistBins)] = hist[ww][x % kHistBins];
        }
    }
}

hipError_t launch_attn_prefill(const AttnArgs& a, hipStream_t s) {
    ProfScope ps("full_attn_prefill", s);
    const int nqt = (a.Tq + kPfWaves - 1) / kPfWaves;
    dim3 grid(a.B * nqt);
    if (a.kv_dtype == HS2_FP8_E4M3) {
        if (a.d == 128) attn_prefill_kernel<128, HS2_FP8_E4M3><<<grid, kPfThreads, 0, s>>>(a);
        else attn_prefill_kernel<64, HS2_FP8_E4M3><<<grid, kPfThreads, 0, s>>>(a);
    } else {
        if (a.d == 128) attn_prefill_kernel<128, HS2_BF16><<<grid, kPfThreads, 0, s>>>(a);
        else attn_prefill_kernel<64, HS2_BF16><<<grid, kPfThreads, 0, s>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_score_prefill(const ScoreArgs& a, hipStream_t s) {
    ProfScope ps("score_prefill", s);
    const int nqt = (a.Tq + kPfWaves - 1) / kPfWaves;
    dim3 grid(a.B * nqt);
    if (a.kv_dtype == HS2_FP8_E4M3) {
        if (a.d == 128) score_prefill_kernel<128, HS2_FP8_E4M3><<<grid, kPfThreads, 0, s>>>(a);
        else score_prefill_kernel<64, HS2_FP8_E4M3><<<grid, kPfThreads, 0, s>>>(a);
    } else {
        if (a.d == 128) score_prefill_kernel<128, HS2_BF16><<<grid, kPfThreads, 0, s>>>(a);
        else score_prefill_kernel<64, HS2_BF16><<<grid, kPfThreads, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace hs2
