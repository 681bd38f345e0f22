// MFMA kernels for query chunks (prefill): the full-attention pass and the score pass.
//
// A chunk of new tokens attends causally over the cache (agentik-os article, section 1: a long
// observation is prefilled into a growing context).  MQA lets the eight query tokens of a
// workgroup share every K/V tile: the tile is read from memory once into LDS and all eight
// waves (one query token each, its 32 heads as the MFMA N dimension) multiply against it.
//
// Pass 1 per wave and 64-key stage:
//   S^T = K_stage . Q^T (bf16 MFMA), causal mask key <= t, online softmax in base 2,
//   O^T += V^T . P^T with V^T built in LDS as fp16 and P rounded to fp16 (fp16 MFMA).
// Pass 2 (score) per wave and 32-key tile:
//   S = Q . K_tile^T, score(j) = sum_h 2^(x_h(j) - lse_h), a per-row radix histogram in LDS.
//
// The cooperative global loads of the next tiles are kept in flight in registers
// (unconditional, clamped loads) while a tile is computed.
#include "mfma_tiles.h"

namespace hs2 {

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;

constexpr int kPfWaves = 8;                  // query tokens (waves) per workgroup
constexpr int kPfThreads = kPfWaves * 64;

// Geometry of the cooperative loads of one 32-row tile in storage format by NT threads.
template <int D, int KV, int NT>
struct PfGeom {
    using G = RawGeom<D, KV>;
    static constexpr int CHUNKS = kTileRows * G::CPR;                    // 16-byte chunks per tile
    static constexpr int NX = (CHUNKS + NT - 1) / NT;                    // loads per thread
};

// Per-thread part of the cooperative tile loads: load x of a thread reads 16-byte chunk c of tile
// row R, at byte offset (k0 + R) * RB + 16 c from the sequence's first cache row.  Offsets are
// 32-bit (the host keeps Nmax * row bytes below 2^31).
template <int D, int KV, int NT>
struct PfLoader {
    using G = RawGeom<D, KV>;
    using P = PfGeom<D, KV, NT>;
    uint32_t off[P::NX];      // R * RB + 16 c
    int R[P::NX];
    __device__ __forceinline__ explicit PfLoader(int tid) {
#pragma unroll
        for (int x = 0; x < P::NX; ++x) {
            int q = tid + x * NT;
            q = q < P::CHUNKS ? q : P::CHUNKS - 1;
            R[x] = q / G::CPR;
            off[x] = (uint32_t)(R[x] * G::RB + 16 * (q % G::CPR));
        }
    }
    // rows k0 .. k0+31, rows at or past khi read row khi - 1 instead; no branch, so the loads can
    // be scheduled among other work
    __device__ __forceinline__ void load_clamped(u32x4_t* raw, const char* seq, int64_t k0, int64_t khi) const {
        const uint32_t lim = (uint32_t)(khi - 1), kb = (uint32_t)k0;
#pragma unroll
        for (int x = 0; x < P::NX; ++x) {
            const uint32_t key = kb + R[x] < lim ? kb + R[x] : lim;
            raw[x] = *(const u32x4_t*)(seq + (key * G::RB + (off[x] - (uint32_t)R[x] * G::RB)));
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

// Byte offset of 16-byte chunk `chunk` of LDS tile row `row`: the swizzled LdsTile layout
// (ST = 0) or rows padded to a stride of ST bytes.
template <int D, int ST>
__device__ __forceinline__ int pf_koff(int row, int chunk) {
    if (ST > 0) return row * ST + 16 * chunk;
    return LdsTile<D>::off(row, chunk);
}

// bf16 LDS tile from raw K (FP8 codes converted exactly).
template <int D, int KV, int NT, int ST>
__device__ __forceinline__ void pf_store_k(const u32x4_t* raw, char* lds, int tid) {
    using G = RawGeom<D, KV>;
    using P = PfGeom<D, KV, NT>;
#pragma unroll
    for (int x = 0; x < P::NX; ++x) {
        const int q = tid + x * NT;
        if (q >= P::CHUNKS) continue;
        const int R = q / G::CPR, c = q % G::CPR;
        if (KV == HS2_FP8_E4M3) {
            u32x4_t lo, hi;
            const u32x2_t a = fp8x4_to_bf16x4(raw[x][0]), b = fp8x4_to_bf16x4(raw[x][1]);
            const u32x2_t cc = fp8x4_to_bf16x4(raw[x][2]), d = fp8x4_to_bf16x4(raw[x][3]);
            lo[0] = a[0]; lo[1] = a[1]; lo[2] = b[0]; lo[3] = b[1];
            hi[0] = cc[0]; hi[1] = cc[1]; hi[2] = d[0]; hi[3] = d[1];
            *(u32x4_t*)(lds + pf_koff<D, ST>(R, 2 * c)) = lo;
            *(u32x4_t*)(lds + pf_koff<D, ST>(R, 2 * c + 1)) = hi;
        } else {
            *(u32x4_t*)(lds + pf_koff<D, ST>(R, c)) = raw[x];
        }
    }
}

// LDS tiles of the attention pass, rows padded instead of swizzled so that every operand read of
// a stage is one base address plus an immediate offset.
//   K:   key rows, stride 2D + 16 bytes (8 consecutive rows of a b128 read start 4 banks apart).
//   V^T: one row per dim with the sub-tile's 32 keys, stride 80 bytes (the rows of 8 lanes of a
//        b128 read cover disjoint banks).  Keys are stored in the order the P operand uses:
//        within each 16-key step, positions 8 hb + j hold key 8 (j / 4) + 4 hb + j % 4, so a
//        lane's 8 operand values are one 16-byte chunk.
//   The V^T tiles come ready-made from vt_prep_kernel, which writes every 32-key sub-tile of the
//   cache once per call as this LDS image (pad bytes included), so a workgroup copies them in
//   whole 16-byte chunks: no conversion, no transposing reads, no scattered writes per workgroup.
//   (Rows of 64 bytes with the chunks XOR-swizzled instead of padded, 20% fewer bytes to copy,
//   measured 11% slower: the operand reads lose their common base address.)
template <int D>
struct PfTiles {
    static constexpr int KST = 2 * D + 16, VTST = 80;
    static constexpr int KB = kTileRows * KST, VTB = D * VTST;
    static constexpr int VTCH = VTB / 16;        // 16-byte chunks of a V^T image
};

// ---- V^T images -----------------------------------------------------------------------------------
// Sub-tile st (keys 32 st .. 32 st + 31) of sequence b becomes D rows of 80 bytes: row n holds dim n
// of the 32 keys as fp16, in the order the P operand uses (16-byte chunk c = 2 ks + hb holds keys
// 16 ks + 4 hb + {0..3} and 16 ks + 8 + 4 hb + {0..3}), then 16 pad bytes.  Keys at or past the
// sequence's length read its last key (finite data that the softmax weights by zero).  The
// conversion truncates (round toward zero): a bf16 value has 8 significant bits, so it is exact in
// fp16 for |v| in [2^-17, 65504] (down to the fp16 subnormal step 2^-24); smaller magnitudes lose
// less than 2^-24, larger ones clamp to 65504.  FP8 E4M3 codes (magnitudes 2^-9 .. 448) convert
// exactly; their row scales stay with P.
__device__ __forceinline__ uint32_t f16x2_bits(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

template <int D, int KV>
__global__ __launch_bounds__(256) void vt_prep_kernel(AttnArgs a) {
    using TL = PfTiles<D>;
    const int b = blockIdx.y;
    const int64_t st = blockIdx.x;
    const int64_t L = seq_len(a.kv_len, b, a.Nmax);
    const int64_t last = L > 0 ? L - 1 : 0;
    const int64_t rowbase = (int64_t)b * a.Nmax;
    char* img = a.vt_img + ((int64_t)b * a.vt_nsub + st) * TL::VTB;
    for (int q = threadIdx.x; q < TL::VTCH; q += 256) {
        const int c = q / D, n = q % D;            // consecutive threads: consecutive dims of one chunk
        u32x4_t o = u32x4_t{};
        if (c < 4) {
            const int ks = c >> 1, hb = c & 1;
            float f[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                int64_t key = st * kTileRows + 16 * ks + 8 * (j >> 2) + 4 * hb + (j & 3);
                key = key < last ? key : last;
                f[j] = load_elem(a.v, a.kv_dtype == HS2_FP8_E4M3 ? HS2_FP8_E4M3 : HS2_BF16, (rowbase + key) * D + n);
            }
#pragma unroll
            for (int w = 0; w < 4; ++w) o[w] = f16x2_bits(f[2 * w], f[2 * w + 1]);
        }
        *(u32x4_t*)(img + n * TL::VTST + 16 * c) = o;
    }
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

// Two wave groups of four waves share each SIMD pairwise and run half a stage apart: while one
// group multiplies (P.V of the previous stage, then S of the current one) the other runs the
// online softmax of its last S, so the matrix cores and the vector ALUs work at the same time.
// A workgroup barrier closes every half-stage.  Group g loads and stages sub-tile g of every
// stage (its K rows and its ready-made V^T image).
//
// Half-step h, group g, e = h - g:
//   e = 2m:    O += P(m-1).V(m-1) and S(m) = K(m).Q as one software-pipelined MFMA sequence
//              (LDS operands read a few MFMAs ahead); in its middle the group stores its K rows
//              of stage m+1 and issues the loads of stage m+2's K rows and stage m+1's V^T
//              image.  The wave runs at raised priority so that its MFMAs are not starved by the
//              other group's VALU.
//   e = 2m+1:  P(m) = softmax step on S(m), then the V^T image writes of stage m+1.
// Three LDS stage buffers cover a stage's lifetime (K is read during the two halves of its own
// stage, V^T during the next two).  Building V^T inside the workgroup (convert, stage, transposing
// reads, writes) took about 10% of the kernel's time in the softmax half; the images are built
// once per call instead (vt_prep_kernel).
//
// The softmax keeps a lazy reference point per head: the weights 2^(x - ref) of a stage are
// computed against the stored reference and kept if every lane's 32 weights sum to at most
// kPfWeightMax (so P <= 2^8, well inside fp16); only otherwise does it take the stage maximum,
// move the reference and rescale O and l.  The per-stage maximum and rescale are skipped on
// nearly every stage.
constexpr float kPfWeightMax = 256.f;
constexpr int kPfAhead = 4;                 // LDS operand reads in flight ahead of the MFMAs
constexpr int kPfMid = 7;                    // MFMA item after which the next sub-tile is stored

// Waves w and w + 4 of a workgroup run on the same SIMD: the groups are w / 4.
__device__ __forceinline__ int pf_group(int w) { return w >> 2; }
__device__ __forceinline__ int pf_gtid(int w, int lane) { return (w & 3) * 64 + lane; }

template <int D, int KV>
__global__ __launch_bounds__(kPfThreads, 1) void attn_prefill_kernel(AttnArgs a) {
    constexpr int KS = D / 16, NB = D / 32;
    constexpr int NT = kPfThreads / 2;           // threads per wave group
    constexpr int NX = PfGeom<D, KV, NT>::NX;
    constexpr int SUB = 2;                       // 32-key sub-tiles per stage (one per group)
    constexpr int SK = SUB * kTileRows;          // keys per stage
    constexpr int NBUF = 3;                      // LDS stage buffers
    using TL = PfTiles<D>;
    __shared__ __attribute__((aligned(16))) char kt[NBUF][SUB][TL::KB];
    __shared__ __attribute__((aligned(16))) char vt[NBUF][SUB][TL::VTB];
    __shared__ float ks_s[NBUF][SUB][kTileRows], vs_s[NBUF][SUB][kTileRows];
    __shared__ int64_t t_s[kPfWaves];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = lane & 31, hb = lane >> 5;
    const int grp = pf_group(w);
    const int gtid = pf_gtid(w, lane);           // thread index inside the group
    const int nqt = (a.Tq + kPfWaves - 1) / kPfWaves;
    const int b = blockIdx.x / nqt, i0 = (blockIdx.x % nqt) * kPfWaves;
    const int H = a.H;
    const int64_t tmax = pf_rows(a.q_pos, a.kv_len, a.Tq, a.Nmax, b, i0, t_s);
    const int64_t t = t_s[w];
    const int r = b * a.Tq + (i0 + w < a.Tq ? i0 + w : a.Tq - 1);
    const int nstages = __builtin_amdgcn_readfirstlane((int)((tmax + 1 + SK - 1) / SK));
    const int last = __builtin_amdgcn_readfirstlane(t >= 0 ? (int)(t / SK) : -1);   // last stage this wave computes
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
    float m_ref = kNegInf, l_run = 0.f;          // l_run per lane half
    const float sl2 = a.scale_log2;

    if (nstages > 0) {
        const int64_t khi = tmax + 1;
        const char* kseq = (const char*)a.k + rowbase * RawGeom<D, KV>::RB;
        const PfLoader<D, KV, NT> ld(gtid);
        u32x4_t rk[NX];
        // this group's V^T image of a stage: 16-byte chunks gtid + NT x (the last ones clamped)
        constexpr int NXV = (TL::VTCH + NT - 1) / NT;
        u32x4_t rvt[NXV];
        const char* vtseq = a.vt_img + (int64_t)b * a.vt_nsub * TL::VTB;
        float rks = 0.f, rvs = 0.f;
        // this group's sub-tile of a stage, clamped into the key range
        auto load = [&](int stage) {
            const int sg = stage < nstages ? stage : nstages - 1;
            const int64_t k0 = (int64_t)sg * SK + grp * kTileRows;
            ld.load_clamped(rk, kseq, k0, khi);
            if (KV == HS2_FP8_E4M3) {
                const int64_t key = k0 + (gtid & 31);
                const int64_t kc = key < khi ? key : khi - 1;
                rks = a.k_scale[rowbase + kc];
                rvs = a.v_scale[rowbase + kc];
            }
        };
        // the V^T image of a stage is loaded in the multiplying half before it and written at the
        // end of the softmax half before it, where the LDS writes do not lengthen the MFMA half
        auto load_v = [&](int stage) {
            const int sg = stage < nstages ? stage : nstages - 1;
            const char* img = vtseq + (int64_t)(sg * SUB + grp) * TL::VTB;
#pragma unroll
            for (int x = 0; x < NXV; ++x) {
                const int q = gtid + x * NT;
                rvt[x] = *(const u32x4_t*)(img + 16 * (q < TL::VTCH ? q : TL::VTCH - 1));
            }
        };
        auto store_v = [&](int buf) {
#pragma unroll
            for (int x = 0; x < NXV; ++x) {
                const int q = gtid + x * NT;
                if (q < TL::VTCH) *(u32x4_t*)(vt[buf][grp] + 16 * q) = rvt[x];
            }
        };
        auto store = [&](int buf) {
            pf_store_k<D, KV, NT, TL::KST>(rk, kt[buf][grp], gtid);
            if (KV == HS2_FP8_E4M3 && gtid < kTileRows) {
                ks_s[buf][grp][gtid] = rks;
                vs_s[buf][grp][gtid] = rvs;
            }
        };
        f32x16_t sacc[SUB];                      // S of a stage, from its multiply to its softmax
        f16x8_t p[SUB][2];                       // P of a stage, from its softmax to the next multiply
#pragma unroll
        for (int sub = 0; sub < SUB; ++sub) {
            sacc[sub] = f32x16_t{};
            p[sub][0] = f16x8_t{};
            p[sub][1] = f16x8_t{};
        }
        load(0);
        load_v(0);
        store(0);
        store_v(0);
        load(1);
        __syncthreads();
        for (int h = 0; h < 2 * nstages + 2; ++h) {
            const int e = h - grp;
            const int m = e >> 1;
            if (e >= 0 && (e & 1) == 0) {
                // ---- multiply half of stage m ----
                // the multiplying wave issues first on its SIMD (otherwise the older wave of the
                // pair wins the arbitration whatever it runs, and the other group's MFMAs starve)
                __builtin_amdgcn_s_setprio(2);
                // One software-pipelined sequence of up to 32 MFMAs: item i < NPV is
                // O^T[dv][head] += V^T . P^T for (blk, sub, ks) = i, item NPV + j is k-step j of
                // S^T = K . Q^T; each item's LDS operand is read kPfAhead items ahead.
                const bool do_pv = m >= 1 && m - 1 <= last;
                const bool do_qk = m < nstages && m <= last;
                constexpr int NPV = NB * SUB * 2, NQK = SUB * KS;
                // V (A operand): 8 keys of dim 32 blk + n from the V^T tile; K (B operand): 8
                // consecutive d of key row n
                const char* vtbase = vt[(m + NBUF - 1) % NBUF][0] + n * TL::VTST + 16 * hb;
                const char* kbase = kt[m % NBUF][0] + n * TL::KST + hb * (D / 16) * 16;
                auto rd = [&](int i) -> u32x4_t {
                    if (i < NPV) {
                        const int blk = i % NB, sub = (i / NB) / 2, ks = (i / NB) % 2;
                        return *(const u32x4_t*)(vtbase + sub * TL::VTB + blk * 32 * TL::VTST + 32 * ks);
                    }
                    const int j = i - NPV, sub = j % SUB, st = j / SUB;
                    return *(const u32x4_t*)(kbase + sub * TL::KB + 16 * st);
                };
                auto mma = [&](int it, const u32x4_t& op) {
                    // consecutive items use different accumulators (dependent MFMAs would wait for
                    // each other's results)
                    if (it < NPV) {
                        const int blk = it % NB, sub = (it / NB) / 2, ks = (it / NB) % 2;
                        oacc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            __builtin_bit_cast(f16x8_t, op), p[sub][ks], oacc[blk], 0, 0, 0);
                    } else {
                        const int j = it - NPV, sub = j % SUB, st = j / SUB;
                        sacc[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8_t, op), qop[st], sacc[sub], 0, 0, 0);
                    }
                };
                // items [I0, I1) as one static sequence; after item kPfMid the group stores its
                // sub-tile of stage m + 1 and issues the loads of stage m + 2, and their vector and
                // memory instructions are spread between the remaining MFMAs.  Stage m + 1's buffers
                // are free at this point even past the last stage (the extra stores go unused).
                auto seq = [&](auto pv, auto qk) {
                    constexpr int I0 = decltype(pv)::value ? 0 : NPV;
                    constexpr int I1 = decltype(qk)::value ? NPV + NQK : NPV;
                    constexpr int N = I1 - I0;
                    u32x4_t win[kPfAhead];
                    // LDS instructions per item
                    auto nrd = [](int) { return 1; };
                    int pro = 0;
#pragma unroll
                    for (int i = 0; i < kPfAhead; ++i)
                        if (i < N) {
                            win[i] = rd(I0 + i);
                            pro += nrd(I0 + i);
                        }
                    if (decltype(qk)::value) {
                        sacc[0] = f32x16_t{};
                        sacc[1] = f32x16_t{};
                    }
                    constexpr int MID = N > kPfMid ? kPfMid : N - 1;
#pragma unroll
                    for (int i = 0; i < N; ++i) {
                        const u32x4_t op = win[i % kPfAhead];
                        if (i + kPfAhead < N) win[i % kPfAhead] = rd(I0 + i + kPfAhead);
                        mma(I0 + i, op);
                        if (i == MID) {
                            store((m + 1) % NBUF);
                            load(m + 2);
                            load_v(m + 1);
                        }
                    }
                    // keep the order: the prologue reads, then per item its MFMA followed by the
                    // reads of the item kPfAhead later
#pragma unroll
                    for (int r = 0; r < 2 * kPfAhead; ++r)
                        if (r < pro) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
                    for (int i = 0; i < N; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
                        for (int r = 0; r < 2; ++r)
                            if (i + kPfAhead < N && r < nrd(I0 + i + kPfAhead)) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                        if (i > MID) {
                            // after the store point: a few vector ALU ops, one LDS write and one
                            // global load per MFMA while they last
                            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
                            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                        }
                    }
                };
                if (do_pv && do_qk) seq(std::true_type{}, std::true_type{});
                else if (do_pv) seq(std::true_type{}, std::false_type{});
                else if (do_qk) seq(std::false_type{}, std::true_type{});
                else {
                    store((m + 1) % NBUF);
                    load(m + 2);
                    load_v(m + 1);
                }
            } else if (e >= 0) {
                // ---- softmax half of stage m ----
                if (m < nstages && m <= last) {
                    const int kb = m % NBUF;
                    const int64_t k0 = (int64_t)m * SK;
                    // logits x = s * sc (sc > 0), in place in the accumulators (a copy would cost
                    // a move per value); keys past t are masked in the stage holding t
                    if (KV == HS2_FP8_E4M3) {
#pragma unroll
                        for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
                            for (int i = 0; i < 16; ++i)
                                sacc[sub][i] *= sl2 * ks_s[kb][sub][8 * (i >> 2) + 4 * hb + (i & 3)];
                    }
                    if (k0 + SK - 1 > t) {
                        const int lim = (int)(t - k0);
#pragma unroll
                        for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
                            for (int i = 0; i < 16; ++i)
                                if (kTileRows * sub + 8 * (i >> 2) + 4 * hb + (i & 3) > lim) sacc[sub][i] = kNegInf;
                    }
                    // bf16 path: x is still unscaled, sc is applied inside the exponent
                    const float scl = KV == HS2_FP8_E4M3 ? 1.f : sl2;
                    // weights 2^(x - mr) into the fp16 P operand (times the V row scale for FP8);
                    // returns the lane's fp32 sum of the unscaled weights (l feeds the log-sum-exp
                    // of the selection scores, which needs more than fp16 precision)
                    // (four partial sums, so that the adds do not form one dependent chain of 32)
                    auto weights = [&](float mr) -> float {
                        float ps4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
                            for (int i = 0; i < 16; ++i) {
                                float e2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[sub][i], scl, -mr));
                                ps4[i & 3] += e2;
                                if (KV == HS2_FP8_E4M3) e2 *= vs_s[kb][sub][8 * (i >> 2) + 4 * hb + (i & 3)];
                                p[sub][i >> 3][i & 7] = (_Float16)e2;
                            }
                        return (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]);
                    };
                    // the reference stays while every lane's weights sum to at most kPfWeightMax;
                    // otherwise (and on the wave's first stage) it moves to the running maximum
                    // and O and l are rescaled
                    bool slow = m_ref == kNegInf;
                    float ps = 0.f;
                    if (!__builtin_amdgcn_ballot_w64(slow)) {
                        ps = weights(m_ref);
                        slow = !(ps <= kPfWeightMax);    // also catches an overflow to inf
                    }
                    if (__builtin_amdgcn_ballot_w64(slow)) {
                        float mt = sacc[0][0];
#pragma unroll
                        for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
                            for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[sub][i]);
                        const float mn = fmaxf(m_ref, pf_half_max(mt) * scl);
                        // exp2(-inf) = 0 clears nothing that is not already zero on a head's
                        // first stage; while a head has seen only masked keys (mn = -inf) the
                        // reference point is 0, never -inf - (-inf)
                        const float alpha = mn == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_ref - mn);
                        m_ref = mn;
                        l_run *= alpha;
#pragma unroll
                        for (int blk = 0; blk < NB; ++blk)
#pragma unroll
                            for (int i = 0; i < 16; ++i) oacc[blk][i] *= alpha;
                        ps = weights(mn == kNegInf ? 0.f : mn);
                    }
                    l_run += ps;
                }
                if (m + 1 < nstages) store_v((m + 1) % NBUF);
            }
            __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
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
            if (hb == 0 && a.lse) a.lse[(int64_t)r * H + n] = l_run > 0.f ? m_ref + log2f(l_run) : kNegInf;
        }
    }
}

// Maximum over the 64 lanes of a wave of values that are >= 0 or negative markers that are all
// equal, in vector registers only: row rotations and quad permutations (DPP) within each 16-lane
// row, then the 16- and 32-lane swaps across rows.  For such values the signed integer order of
// the bit patterns is the float order, so one integer max per step does the work (a float max
// costs three here: the compiler canonicalises both operands first).
__device__ __forceinline__ float pf_wave_max_nonneg(float v) {
    int x = __float_as_int(v);
    x = max(x, __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, true));   // row_ror:8
    x = max(x, __builtin_amdgcn_mov_dpp(x, 0x124, 0xF, 0xF, true));   // row_ror:4
    x = max(x, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true));    // quad [2,3,0,1]
    x = max(x, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true));    // quad [1,0,3,2]
    const auto p = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
    x = max((int)p[0], (int)p[1]);
    const auto q = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
    return __int_as_float(max((int)q[0], (int)q[1]));
}

// ---- pass 2: selection scores ---------------------------------------------------------------------
// 64-key stages (two 32-key sub-tiles) in three LDS buffers, software-pipelined per wave: the
// MFMAs of stage m + 1 are interleaved with the exponentials of stage m, so the matrix cores and
// the vector ALUs of a wave work at the same time.  One barrier per stage.
constexpr int kScoreAhead = 4;               // LDS operand reads in flight ahead of the MFMAs
template <int D, int KV>
__global__ __launch_bounds__(kPfThreads, 1) void score_prefill_kernel(ScoreArgs a) {
    constexpr int KS = D / 16;
    constexpr int NX = PfGeom<D, KV, kPfThreads>::NX;
    constexpr int SUB = 2, SK = SUB * kTileRows, NBUF = 3;
    // K rows padded to PfTiles<D>::KST bytes, as in the attention pass: every operand read of a
    // stage is one base address plus an immediate offset (a swizzled tile needs an address
    // computation per read)
    using TL = PfTiles<D>;
    __shared__ __attribute__((aligned(16))) char kt[NBUF][SUB][TL::KB];
    __shared__ float ks_s[NBUF][SUB][kTileRows];
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
    const int nstages = __builtin_amdgcn_readfirstlane((int)((Cmax + SK - 1) / SK));
    const int last = __builtin_amdgcn_readfirstlane(C > 0 ? (int)((C - 1) / SK) : -1);   // last stage with candidates
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

    if (nstages > 0) {
        const char* kseq = (const char*)a.k + rowbase * RawGeom<D, KV>::RB;
        const PfLoader<D, KV, kPfThreads> ld(threadIdx.x);
        // two register stages: stage s is loaded into registers s % 2 two iterations before it
        // is stored to LDS
        u32x4_t rk[2][SUB][NX];
        float rks[2][SUB];
        auto load = [&](int stage) {
            const int sg = stage < nstages ? stage : nstages - 1;
            const int rs = stage & 1;
#pragma unroll
            for (int sub = 0; sub < SUB; ++sub) {
                const int64_t k0 = (int64_t)sg * SK + sub * kTileRows;
                ld.load_clamped(rk[rs][sub], kseq, k0, Cmax);
                if (KV == HS2_FP8_E4M3) {
                    const int64_t key = k0 + (threadIdx.x & 31);
                    rks[rs][sub] = a.k_scale[rowbase + (key < Cmax ? key : Cmax - 1)];
                }
            }
        };
        auto store = [&](int stage) {
            const int buf = stage % NBUF, rs = stage & 1;
#pragma unroll
            for (int sub = 0; sub < SUB; ++sub) {
                pf_store_k<D, KV, kPfThreads, TL::KST>(rk[rs][sub], kt[buf][sub], threadIdx.x);
                if (KV == HS2_FP8_E4M3 && threadIdx.x < kTileRows) ks_s[buf][sub][threadIdx.x] = rks[rs][sub];
            }
        };
        // S = Q . K^T of a stage's sub-tiles: lane (key n, half hb) holds heads 8 (i / 4) + 4 hb + i % 4
        auto mma = [&](f32x16_t* sacc, int buf) {
#pragma unroll
            for (int sub = 0; sub < SUB; ++sub) {
                sacc[sub] = f32x16_t{};
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    sacc[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        qop[s], *(const bf16x8_t*)(kt[buf][sub] + n * TL::KST + (hb * (D / 16) + s) * 16), sacc[sub], 0, 0, 0);
            }
        };
        const int klane = n * TL::KST + hb * (D / 16) * 16;   // this lane's operand row and half
        f32x16_t sa[SUB], sb[SUB];            // S of consecutive stages (even / odd)
        load(0);
        store(0);
        if (nstages > 1) {
            load(1);
            store(1);
        }
        load(2);
        load(3);
        __syncthreads();
        mma(sa, 0);
        // iteration m: the scores of stage m and the MFMAs of stage m + 1 in one branch-free block
        // (MFMAs past the last stage read a stale buffer and their results go unused), then the
        // stores of stage m's scores, stage m + 2 into LDS and the loads of stage m + 4.
        // Iterations come in pairs that always run both halves, and the LDS store of stage m + 2 is
        // unconditional (past the last stage the clamped loads hold the last stage again, written
        // into a buffer no later MFMA of a live stage reads): the loop then has one back edge with
        // one set of loads in flight, and the compiler's wait before that store covers only the
        // loads of stage m + 2, not those of stage m + 3 issued one iteration later.
        auto iter = [&](int m, f32x16_t* cur, f32x16_t* nxt) {
            // One static sequence of SUB * KS steps.  Step i issues MFMA i of stage m + 1 (k-step
            // i / SUB of sub-tile i % SUB, so consecutive MFMAs use different accumulators), the LDS
            // read of the operand kScoreAhead steps later, and EPS of the lane's 32 exponentials of
            // stage m (sub-tile v / 16, head slot v % 16 for v = EPS i .. EPS i + EPS - 1; EPS = 2
            // at d = 128, 4 at d = 64).  A scheduling barrier
            // closes every step: without it the compiler issued all MFMAs, each behind its own
            // operand read, and then all exponentials, so a wave's MFMAs and vector work did not
            // overlap.  Each sum keeps its order (head slots 0..15), so results do not change.
            constexpr int NM = SUB * KS;
            constexpr int EPS = SUB * 16 / NM;       // exponentials per step
            static_assert(EPS * NM == SUB * 16, "every exponential belongs to one step");
            const int mb = (m + 1) % NBUF;
            float sc[SUB];
#pragma unroll
            for (int sub = 0; sub < SUB; ++sub) {
                sc[sub] = a.scale_log2;
                if (KV == HS2_FP8_E4M3) sc[sub] *= ks_s[m % NBUF][sub][n];
            }
            // one scalar buffer offset plus the lane's fixed offset; the reads differ by immediates
            const int boff = __builtin_amdgcn_readfirstlane(mb * (SUB * TL::KB));
            const char* kbase = &kt[0][0][0] + boff + klane;
            auto rd = [&](int i) { return *(const bf16x8_t*)(kbase + (i % SUB) * TL::KB + (i / SUB) * 16); };
            bf16x8_t win[kScoreAhead];
#pragma unroll
            for (int i = 0; i < kScoreAhead; ++i) win[i] = rd(i);
            float x[SUB] = {0.f, 0.f};
#pragma unroll
            for (int sub = 0; sub < SUB; ++sub) nxt[sub] = f32x16_t{};
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                const bf16x8_t op = win[i % kScoreAhead];
                if (i + kScoreAhead < NM) win[i % kScoreAhead] = rd(i + kScoreAhead);
                nxt[i % SUB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qop[i / SUB], op, nxt[i % SUB], 0, 0, 0);
#pragma unroll
                for (int u = 0; u < EPS; ++u) {
                    const int v = EPS * i + u, vs = v / 16, e = v % 16;
                    x[vs] += __builtin_amdgcn_exp2f(__builtin_fmaf(cur[vs][e], sc[vs], nlse[e]));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // score(j) = sum_h 2^(x_h(j) - lse_h): 16 heads per lane, the partner lane's 16
            // through v_permlane32_swap
            float acc[SUB];
#pragma unroll
            for (int sub = 0; sub < SUB; ++sub) acc[sub] = pf_half_sum(x[sub]);
            if (m <= last) {
                // both lane halves hold both sums: lane (n, hb) stores key n of sub-tile hb
                const float v = hb ? acc[1] : acc[0];
                const int64_t j = (int64_t)m * SK + hb * kTileRows + n;
                if (a.bscore) {
                    // block selection with 64-key blocks: lane l holds key 64 m + l, so the stage's
                    // block maximum is the wave's (scores are >= 0; -1 marks a key past C)
                    const float bm = pf_wave_max_nonneg(j < C ? v : -1.0f);
                    if (lane == 0) a.bscore[(int64_t)r * a.bstride + m] = bm;
                } else if (j < C) {
                    srow[j] = v;
                    atomicAdd(&hist[w][__float_as_uint(v) >> 21], 1u);
                }
            }
            store(m + 2);
            load(m + 4);
            __syncthreads();
        };
        for (int m = 0; m < nstages; m += 2) {
            iter(m, sa, sb);
            iter(m + 1, sb, sa);
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

// V^T images of every sequence's cache (vt_nsub sub-tiles each), then the attention pass.
hipError_t launch_attn_prefill(const AttnArgs& a, hipStream_t s) {
    {
        ProfScope ps("vt_prep", s);
        dim3 grid((unsigned)a.vt_nsub, a.B);
        if (a.kv_dtype == HS2_FP8_E4M3) {
            if (a.d == 128) vt_prep_kernel<128, HS2_FP8_E4M3><<<grid, 256, 0, s>>>(a);
            else vt_prep_kernel<64, HS2_FP8_E4M3><<<grid, 256, 0, s>>>(a);
        } else {
            if (a.d == 128) vt_prep_kernel<128, HS2_BF16><<<grid, 256, 0, s>>>(a);
            else vt_prep_kernel<64, HS2_BF16><<<grid, 256, 0, s>>>(a);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
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
