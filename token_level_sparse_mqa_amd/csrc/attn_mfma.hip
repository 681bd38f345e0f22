// MFMA attention kernels for one query row per workgroup (decode rows, sparse rows).
//
// MQA (ainews page, experimental-setup paragraph): all H query heads of a token share one
// K/V row, so a 32-key tile of the cache is read once and multiplied against all heads with
// v_mfma_f32_32x32x16 (heads padded to 32 form the N dimension).  The full layer (causal
// range of keys) and the sparse layers (a list of selected rows: KV Reuse, lynxflow blog
// "Two-Level KV Sharing") share this kernel; only the source of the key ids differs.
//
// Per wave and 32-key tile:
//   S^T[key][head] = K_tile . Q^T          8 (D=128) bf16 MFMAs; lane (n, hb) owns head n
//   online softmax per head in base 2      (x = s * sm * log2 e; 16 keys per lane + partner)
//   O^T[dv][head] += V^T . P^T             P in fp16; V^T staged in LDS as fp16 key pairs
// The four waves of a workgroup take interleaved tiles of the workgroup's key range and are
// merged in LDS; several workgroups per row (splits) are merged by attn_split_combine.
//
// The d-index order inside the QK product is free (both operands use it): lane half hb
// covers d in [hb*D/2, hb*D/2 + D/2), eight consecutive values per k-step, so every lane
// reads one contiguous half row of K.  The key order inside the PV product is likewise
// free; it follows the S^T register layout so P needs no shuffles.
//
// FP8 caches (OCP E4M3FN + per-row fp32 scale): codes are converted exactly to bf16 (K) and
// fp16 (V); the K scale multiplies the logits of its key, the V scale multiplies P.
#include "hs2_device.h"

namespace hs2 {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

constexpr int kRowWaves = 4;
constexpr int kVtRow = 18;          // dwords per V^T row in LDS: 16 key pairs + 2 pad

// ---- conversions -------------------------------------------------------------------------------

// Two E4M3FN codes (byte 0/1 or 2/3 of w) -> two fp32 (exact).
template <bool HI>
__device__ __forceinline__ f32x2_t fp8x2_to_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}

// Upper halves of two fp32 -> packed bf16 pair (exact when the values are bf16-representable).
__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Eight E4M3 codes (two dwords) -> eight bf16 as an MFMA operand.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
    u32x4_t r;
    f32x2_t a = fp8x2_to_f32<false>(w0), b = fp8x2_to_f32<true>(w0);
    f32x2_t c = fp8x2_to_f32<false>(w1), d = fp8x2_to_f32<true>(w1);
    r[0] = pack_hi16(a[0], a[1]);
    r[1] = pack_hi16(b[0], b[1]);
    r[2] = pack_hi16(c[0], c[1]);
    r[3] = pack_hi16(d[0], d[1]);
    return __builtin_bit_cast(bf16x8_t, r);
}

__device__ __forceinline__ uint32_t f16x2_bits(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// Round-to-nearest fp32 -> fp16 for the attention weights.
__device__ __forceinline__ f16x8_t to_f16x8(const float* x) {
    f16x8_t r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (_Float16)x[e];
    return r;
}

// ---- raw tile data held in registers -------------------------------------------------------------
template <int D, int KV>
struct RowTile {
    static constexpr int KB = KV == HS2_FP8_E4M3 ? D / 32 : D / 16;   // u32x4 of K per lane
    static constexpr int VB = KV == HS2_FP8_E4M3 ? D / 64 : D / 32;   // u32x4 of V per key, 2 keys
    u32x4_t k[KB];
    u32x4_t v[2][VB];
    int32_t kid;          // key id of S^T row (lane & 31); -1 = none
    float ks, vs;         // fp8 scales of that row
};

template <int D, int KV>
__device__ __forceinline__ void load_row_tile(RowTile<D, KV>& T, const AttnArgs& a, int b, int64_t L,
                                              int64_t e_lo, int64_t e_hi, int64_t tile_e, int r) {
    const int lane = threadIdx.x & 63;
    const int m = lane & 31, hb = lane >> 5;
    const int64_t e = tile_e + m;
    int64_t j = -1;
    if (e < e_hi && e >= e_lo) {
        j = a.list ? (int64_t)a.list[(int64_t)r * a.S + e] : e;
        if (j < 0 || j >= L) j = -1;
    }
    T.kid = (int32_t)j;
    const int64_t row = (int64_t)b * a.Nmax + (j < 0 ? 0 : j);
    constexpr int ESZ = KV == HS2_FP8_E4M3 ? 1 : 2;
    const u32x4_t* kp = (const u32x4_t*)((const char*)a.k + (row * D + hb * (D / 2)) * ESZ);
#pragma unroll
    for (int x = 0; x < RowTile<D, KV>::KB; ++x) T.k[x] = j >= 0 ? kp[x] : u32x4_t{0, 0, 0, 0};
    if (KV == HS2_FP8_E4M3) {
        T.ks = j >= 0 ? a.k_scale[row] : 0.f;
        T.vs = j >= 0 ? a.v_scale[row] : 0.f;
    }
    // V: this lane loads keys 2p, 2p+1 (p = lane & 15), dims [g*D/4, g*D/4 + D/4) (g = lane >> 4)
    const int p = lane & 15, g = lane >> 4;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int32_t jj = __shfl(T.kid, 2 * p + u);
        const int64_t vrow = (int64_t)b * a.Nmax + (jj < 0 ? 0 : jj);
        const u32x4_t* vp = (const u32x4_t*)((const char*)a.v + (vrow * D + g * (D / 4)) * ESZ);
#pragma unroll
        for (int x = 0; x < RowTile<D, KV>::VB; ++x) T.v[u][x] = jj >= 0 ? vp[x] : u32x4_t{0, 0, 0, 0};
    }
}

// Write the V tile of this wave transposed into LDS as fp16 pairs: vt[dv * kVtRow + p] holds
// (V[2p][dv], V[2p+1][dv]).
template <int D, int KV>
__device__ __forceinline__ void store_vt(const RowTile<D, KV>& T, uint32_t* vt) {
    const int lane = threadIdx.x & 63;
    const int p = lane & 15, g = lane >> 4;
    uint32_t* dst = vt + (g * (D / 4)) * kVtRow + p;
    if (KV == HS2_FP8_E4M3) {
        // D/4 codes per key in VB u32x4 (16 codes each)
#pragma unroll
        for (int x = 0; x < RowTile<D, KV>::VB; ++x)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const f32x2_t a0 = fp8x2_to_f32<false>(T.v[0][x][w]), a1 = fp8x2_to_f32<false>(T.v[1][x][w]);
                const f32x2_t b0 = fp8x2_to_f32<true>(T.v[0][x][w]), b1 = fp8x2_to_f32<true>(T.v[1][x][w]);
                const int c = x * 16 + w * 4;
                dst[(c + 0) * kVtRow] = f16x2_bits(a0[0], a1[0]);
                dst[(c + 1) * kVtRow] = f16x2_bits(a0[1], a1[1]);
                dst[(c + 2) * kVtRow] = f16x2_bits(b0[0], b1[0]);
                dst[(c + 3) * kVtRow] = f16x2_bits(b0[1], b1[1]);
            }
    } else {
#pragma unroll
        for (int x = 0; x < RowTile<D, KV>::VB; ++x)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t u0 = T.v[0][x][w], u1 = T.v[1][x][w];
                const int c = x * 8 + w * 2;
                dst[(c + 0) * kVtRow] = f16x2_bits(__uint_as_float(u0 << 16), __uint_as_float(u1 << 16));
                dst[(c + 1) * kVtRow] = f16x2_bits(__uint_as_float(u0 & 0xffff0000u), __uint_as_float(u1 & 0xffff0000u));
            }
    }
}

template <int D, int KV>
__device__ __forceinline__ bf16x8_t k_operand(const RowTile<D, KV>& T, int s) {
    if (KV == HS2_FP8_E4M3) {
        const u32x4_t w = T.k[s >> 1];
        return (s & 1) ? fp8x8_to_bf16x8(w[2], w[3]) : fp8x8_to_bf16x8(w[0], w[1]);
    }
    return __builtin_bit_cast(bf16x8_t, T.k[s]);
}

__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// ---- the attention kernel -------------------------------------------------------------------------
template <int D, int KV>
__global__ __launch_bounds__(256) void attn_rows_mfma_kernel(AttnArgs a) {
    constexpr int KS = D / 16;
    constexpr int NB = D / 32;
    __shared__ uint32_t vt_all[kRowWaves][D * kVtRow];
    __shared__ float ml_s[kRowWaves][32][2];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = lane & 31, hb = lane >> 5;
    const int r = blockIdx.x, split = blockIdx.y;
    const int b = r / a.Tq;
    const int H = a.H;
    const int64_t L = seq_len(a.kv_len, b, a.Nmax);
    int64_t e0 = (int64_t)split * a.chunk, e1;
    if (a.list) {
        e1 = e0 + a.chunk < a.S ? e0 + a.chunk : a.S;
    } else {
        const int64_t t = row_pos(a.q_pos, a.kv_len, r, a.Tq, a.Nmax);
        e1 = e0 + a.chunk < t + 1 ? e0 + a.chunk : t + 1;
    }
    const int64_t ntiles = e1 > e0 ? (e1 - e0 + 31) / 32 : 0;

    // Q^T operand: head n, d in [hb*D/2 + 8s, +8)
    bf16x8_t qop[KS];
    {
        const u32x4_t* qp = (const u32x4_t*)((const uint16_t*)a.q + ((int64_t)r * H + (n < H ? n : 0)) * D + hb * (D / 2));
#pragma unroll
        for (int s = 0; s < KS; ++s) qop[s] = n < H ? __builtin_bit_cast(bf16x8_t, qp[s]) : bf16x8_t{};
    }
    uint32_t* vt = vt_all[w];
    f32x16_t oacc[NB];
#pragma unroll
    for (int x = 0; x < NB; ++x) oacc[x] = f32x16_t{};
    float m_run = kNegInf, l_run = 0.f;
    const float sl2 = a.scale_log2;

    RowTile<D, KV> cur, nxt;
    int64_t tile = w;
    if (tile < ntiles) load_row_tile<D, KV>(cur, a, b, L, e0, e1, e0 + 32 * tile, r);
    for (; tile < ntiles; tile += kRowWaves) {
        const int64_t nt = tile + kRowWaves;
        if (nt < ntiles) load_row_tile<D, KV>(nxt, a, b, L, e0, e1, e0 + 32 * nt, r);

        store_vt<D, KV>(cur, vt);
        f32x16_t sacc = f32x16_t{};
#pragma unroll
        for (int s = 0; s < KS; ++s)
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_operand<D, KV>(cur, s), qop[s], sacc, 0, 0, 0);
        // logits of keys m_i = 8(i/4) + 4hb + i%4 for head n
        float x[16];
        float mt = kNegInf;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = 8 * (i >> 2) + 4 * hb + (i & 3);
            const int32_t kid = __shfl(cur.kid, m);
            float sc = sl2;
            if (KV == HS2_FP8_E4M3) sc *= __shfl(cur.ks, m);
            x[i] = kid >= 0 ? sacc[i] * sc : kNegInf;
            mt = fmaxf(mt, x[i]);
        }
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mn = fmaxf(m_run, mt);
        const float alpha = (mn == kNegInf) ? 1.f : exp2f(m_run - mn);
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            x[i] = (x[i] == kNegInf) ? 0.f : exp2f(x[i] - mn);
            ps += x[i];
        }
        ps += __shfl_xor(ps, 32);
        l_run = l_run * alpha + ps;
        m_run = mn;
        if (KV == HS2_FP8_E4M3) {
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] *= __shfl(cur.vs, 8 * (i >> 2) + 4 * hb + (i & 3));
        }
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[blk][i] *= alpha;
        const f16x8_t p0 = to_f16x8(&x[0]), p1 = to_f16x8(&x[8]);
        wave_lds_fence();
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            const uint32_t* row = vt + (blk * 32 + n) * kVtRow;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                u32x4_t av;
                const u32x2_t lo = *(const u32x2_t*)(row + 8 * ks + 2 * hb);
                const u32x2_t hi = *(const u32x2_t*)(row + 8 * ks + 4 + 2 * hb);
                av[0] = lo[0]; av[1] = lo[1]; av[2] = hi[0]; av[3] = hi[1];
                oacc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, av),
                                                                   ks ? p1 : p0, oacc[blk], 0, 0, 0);
            }
        }
        wave_lds_fence();
        cur = nxt;
    }

    // ---- merge the waves of the workgroup ----
    if (lane < 32) { ml_s[w][n][0] = m_run; ml_s[w][n][1] = l_run; }
    __syncthreads();
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < kRowWaves; ++ww) M = fmaxf(M, ml_s[ww][n][0]);
    float Lsum = 0.f, myscale = 0.f;
#pragma unroll
    for (int ww = 0; ww < kRowWaves; ++ww) {
        const float mw = ml_s[ww][n][0];
        const float sw = (mw == kNegInf) ? 0.f : exp2f(mw - M);
        Lsum += ml_s[ww][n][1] * sw;
        if (ww == w) myscale = sw;
    }
    float* obuf = (float*)&vt_all[0][0];     // [32 heads][D] fp32, reusing the V^T space
    for (int ww = 0; ww < kRowWaves; ++ww) {
        if (w == ww) {
#pragma unroll
            for (int blk = 0; blk < NB; ++blk)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int dv = blk * 32 + 8 * (i >> 2) + 4 * hb + (i & 3);
                    const float v = oacc[blk][i] * myscale;
                    obuf[n * D + dv] = ww == 0 ? v : obuf[n * D + dv] + v;
                }
        }
        __syncthreads();
    }
    // write: all threads over H*D outputs
    for (int x = threadIdx.x; x < H * D; x += 256) {
        const int h = x / D, dv = x % D;
        float Mh = kNegInf, Lh = 0.f;
#pragma unroll
        for (int ww = 0; ww < kRowWaves; ++ww) Mh = fmaxf(Mh, ml_s[ww][h][0]);
#pragma unroll
        for (int ww = 0; ww < kRowWaves; ++ww) {
            const float mw = ml_s[ww][h][0];
            Lh += mw == kNegInf ? 0.f : ml_s[ww][h][1] * exp2f(mw - Mh);
        }
        const float ov = obuf[h * D + dv];
        if (a.part) {
            float* pp = a.part + (((int64_t)r * a.nsplit + split) * H + h) * (D + 2);
            pp[dv] = ov;
            if (dv == 0) { pp[D] = Mh; pp[D + 1] = Lh; }
        } else {
            a.o[((int64_t)r * H + h) * D + dv] = Lh > 0.f ? ov / Lh : 0.f;
            if (dv == 0 && a.lse) a.lse[(int64_t)r * H + h] = Lh > 0.f ? Mh + log2f(Lh) : kNegInf;
        }
    }
    (void)Lsum;
}

// ---- merge of the splits of each row (one workgroup per (row, head)) ------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_split_combine_kernel(AttnArgs a) {
    __shared__ float red[256];
    __shared__ float accs[2][D];
    const int r = blockIdx.x, h = blockIdx.y, H = a.H, ns = a.nsplit;
    const int tid = threadIdx.x;
    const float* base = a.part + ((int64_t)r * ns * H + h) * (D + 2);
    const int64_t sstride = (int64_t)H * (D + 2);
    float m = kNegInf;
    for (int s = tid; s < ns; s += 256) m = fmaxf(m, base[s * sstride + D]);
    red[tid] = m;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
        __syncthreads();
    }
    const float M = red[0];
    __syncthreads();
    float l = 0.f;
    for (int s = tid; s < ns; s += 256) {
        const float ms = base[s * sstride + D];
        if (ms != kNegInf) l += base[s * sstride + D + 1] * exp2f(ms - M);
    }
    red[tid] = l;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) red[tid] += red[tid + o];
        __syncthreads();
    }
    const float Ltot = red[0];
    // output dims: 256 threads = 2 split phases x 128 dims (D = 128) or 4 x 64
    constexpr int PH = 256 / D;
    const int dv = tid % D, ph = tid / D;
    float acc = 0.f;
    if (M != kNegInf) {
        for (int s = ph; s < ns; s += PH) {
            const float* p = base + s * sstride;
            const float ms = p[D];
            if (ms != kNegInf) acc += p[dv] * exp2f(ms - M);
        }
    }
    __syncthreads();
    red[tid] = acc;
    __syncthreads();
    if (ph == 0) {
        float tot = 0.f;
#pragma unroll
        for (int q = 0; q < PH; ++q) tot += red[q * D + dv];
        a.o[((int64_t)r * H + h) * D + dv] = Ltot > 0.f ? tot / Ltot : 0.f;
        if (dv == 0 && a.lse) a.lse[(int64_t)r * H + h] = Ltot > 0.f ? M + log2f(Ltot) : kNegInf;
    }
    (void)accs;
}

// ---- score pass --------------------------------------------------------------------------------
// score(j) = sum_h 2^(x_h(j) - lse_h) for candidates j in [0, t - window]; S[head][key] = Q . K^T
// so that every lane owns one key and sums its 16 heads, plus the partner lane's 16.
template <int D, int KV>
__global__ __launch_bounds__(256) void score_rows_mfma_kernel(ScoreArgs a) {
    constexpr int KS = D / 16;
    constexpr int KB = KV == HS2_FP8_E4M3 ? D / 32 : D / 16;
    constexpr int ESZ = KV == HS2_FP8_E4M3 ? 1 : 2;
    __shared__ uint32_t hist[kHistBins];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = lane & 31, hb = lane >> 5;
    const int r = blockIdx.x, split = blockIdx.y;
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

    bf16x8_t qop[KS];
    {
        const u32x4_t* qp = (const u32x4_t*)((const uint16_t*)a.q + ((int64_t)r * H + (n < H ? n : 0)) * D + hb * (D / 2));
#pragma unroll
        for (int s = 0; s < KS; ++s) qop[s] = n < H ? __builtin_bit_cast(bf16x8_t, qp[s]) : bf16x8_t{};
    }
    // negative base-2 log normaliser of the 16 heads this lane sums: heads 8(i/4) + 4hb + i%4
    float nlse[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int h = 8 * (i >> 2) + 4 * hb + (i & 3);
        nlse[i] = h < H ? -a.lse[(int64_t)r * H + h] : kNegInf;
    }
    if (a.rowhist) __syncthreads();

    u32x4_t kc[KB], kn[KB];
    float ksc = 1.f, ksn = 1.f;
    auto load = [&](u32x4_t* kr, float& ks, int64_t tl) {
        const int64_t j = e0 + 32 * tl + n;
        const bool ok = j < e1;
        const int64_t row = (int64_t)b * a.Nmax + (ok ? j : 0);
        const u32x4_t* kp = (const u32x4_t*)((const char*)a.k + (row * D + hb * (D / 2)) * ESZ);
#pragma unroll
        for (int x = 0; x < KB; ++x) kr[x] = ok ? kp[x] : u32x4_t{0, 0, 0, 0};
        if (KV == HS2_FP8_E4M3) ks = ok ? a.k_scale[row] : 0.f;
    };
    int64_t tile = w;
    if (tile < ntiles) load(kc, ksc, tile);
    float* srow = a.scores + (int64_t)r * a.cstride;
    for (; tile < ntiles; tile += kRowWaves) {
        const int64_t nt = tile + kRowWaves;
        if (nt < ntiles) load(kn, ksn, nt);
        f32x16_t sacc = f32x16_t{};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            bf16x8_t kop;
            if (KV == HS2_FP8_E4M3) {
                const u32x4_t ww = kc[s >> 1];
                kop = (s & 1) ? fp8x8_to_bf16x8(ww[2], ww[3]) : fp8x8_to_bf16x8(ww[0], ww[1]);
            } else {
                kop = __builtin_bit_cast(bf16x8_t, kc[s]);
            }
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qop[s], kop, sacc, 0, 0, 0);
        }
        float sc = a.scale_log2;
        if (KV == HS2_FP8_E4M3) sc *= ksc;
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc += exp2f(sacc[i] * sc + nlse[i]);
        acc += __shfl_xor(acc, 32);
        const int64_t j = e0 + 32 * tile + n;
        if (hb == 0 && j < e1) {
            srow[j] = acc;
            if (a.rowhist) atomicAdd(&hist[__float_as_uint(acc) >> 21], 1u);
        }
#pragma unroll
        for (int x = 0; x < KB; ++x) kc[x] = kn[x];
        ksc = ksn;
    }
    if (a.rowhist) {
        __syncthreads();
        for (int x = threadIdx.x; x < kHistBins; x += 256)
            if (hist[x]) atomicAdd(&a.rowhist[(int64_t)r * kHistBins + x], hist[x]);
    }
}

// ---- launchers -------------------------------------------------------------------------------------
hipError_t launch_attn_rows_mfma(const AttnArgs& a, const char* name, hipStream_t s) {
    ProfScope ps(name, s);
    dim3 grid(a.B * a.Tq, a.nsplit);
    if (a.kv_dtype == HS2_FP8_E4M3) {
        if (a.d == 128) attn_rows_mfma_kernel<128, HS2_FP8_E4M3><<<grid, 256, 0, s>>>(a);
        else attn_rows_mfma_kernel<64, HS2_FP8_E4M3><<<grid, 256, 0, s>>>(a);
    } else {
        if (a.d == 128) attn_rows_mfma_kernel<128, HS2_BF16><<<grid, 256, 0, s>>>(a);
        else attn_rows_mfma_kernel<64, HS2_BF16><<<grid, 256, 0, s>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_attn_split_combine(const AttnArgs& a, const char* name, hipStream_t s) {
    ProfScope ps(name, s);
    dim3 grid(a.B * a.Tq, a.H);
    if (a.d == 128) attn_split_combine_kernel<128><<<grid, 256, 0, s>>>(a);
    else attn_split_combine_kernel<64><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_score_rows_mfma(const ScoreArgs& a, hipStream_t s) {
    ProfScope ps("score_rows_mfma", s);
    dim3 grid(a.B * a.Tq, a.nsplit);
    if (a.kv_dtype == HS2_FP8_E4M3) {
        if (a.d == 128) score_rows_mfma_kernel<128, HS2_FP8_E4M3><<<grid, 256, 0, s>>>(a);
        else score_rows_mfma_kernel<64, HS2_FP8_E4M3><<<grid, 256, 0, s>>>(a);
    } else {
        if (a.d == 128) score_rows_mfma_kernel<128, HS2_BF16><<<grid, 256, 0, s>>>(a);
        else score_rows_mfma_kernel<64, HS2_BF16><<<grid, 256, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace hs2
