// Generic attention kernels (VALU, fp32 arithmetic) for every supported dtype and shape.
//
// They carry the fp32 path (fp32 Q/K/V) and serve any shape the MFMA kernels do not cover.
// One workgroup handles one query row (all H heads of one query token, sharing the single
// KV head: MQA) over one split of its key set; splits are merged by attn_combine.
//
// Arithmetic, per query row and head h (agentik-os article, section 2: the full layer and the
// sparse layers of a hybrid block attend over one shared cache):
//   x_h(j) = (sm * log2 e) * q_h . k_j          (base-2 logits)
//   m_h = max_j x_h(j),  l_h = sum_j 2^(x_h(j) - m_h),  o_h = sum_j 2^(x_h(j) - m_h) v_j / l_h
// computed online over key tiles, so that softmax needs one pass over K and V.
#include "hs2_device.h"

namespace hs2 {

constexpr int kGenTile = 32;     // keys per tile
constexpr int kGenThreads = 256;

template <int D>
__global__ __launch_bounds__(kGenThreads) void attn_generic_kernel(AttnArgs a) {
    __shared__ float qs[32][D];
    __shared__ float ks[kGenTile][D + 1];
    __shared__ float vs[kGenTile][D];
    __shared__ float ss[32][kGenTile + 1];
    __shared__ int64_t kid[kGenTile];
    __shared__ float m_s[32], l_s[32], al_s[32];

    const int r = blockIdx.x, split = blockIdx.y, tid = threadIdx.x;
    const int b = r / a.Tq;
    const int H = a.H;
    const int64_t L = seq_len(a.kv_len, b, a.Nmax);

    int64_t e0 = (int64_t)split * a.chunk, e1;
    int64_t t = -1;
    if (a.list) {
        e1 = e0 + a.chunk < a.S ? e0 + a.chunk : a.S;
    } else {
        t = row_pos(a.q_pos, a.kv_len, r, a.Tq, a.Nmax);
        e1 = e0 + a.chunk < t + 1 ? e0 + a.chunk : t + 1;
    }

    // this row's selection workspace is cleared here, before the score pass accumulates into it
    if (a.zero_hist && split == 0) {
        for (int x = tid; x < kHistBins; x += kGenThreads) a.zero_hist[(int64_t)r * kHistBins + x] = 0;
        if (tid < 4) a.zero_cnt[(int64_t)r * 4 + tid] = 0;
    }
    for (int x = tid; x < 32 * D; x += kGenThreads) {
        const int h = x / D, c = x % D;
        qs[h][c] = h < H ? load_elem(a.q, a.q_dtype, ((int64_t)r * H + h) * D + c) * a.scale_log2 : 0.f;
    }
    if (tid < 32) { m_s[tid] = kNegInf; l_s[tid] = 0.f; }

    constexpr int NO = D / 8;        // outputs per thread: head tid/8, dims (tid%8) + 8u
    float oacc[NO];
#pragma unroll
    for (int u = 0; u < NO; ++u) oacc[u] = 0.f;
    const int hh = tid >> 3, dv0 = tid & 7;

    for (int64_t eb = e0; eb < e1; eb += kGenTile) {
        __syncthreads();
        if (tid < kGenTile) {
            const int64_t e = eb + tid;
            int64_t j = -1;
            if (e < e1) {
                j = a.list ? (int64_t)a.list[(int64_t)r * a.S + e] : e;
                if (j < 0 || j >= L) j = -1;
            }
            kid[tid] = j;
        }
        __syncthreads();
        for (int x = tid; x < kGenTile * D; x += kGenThreads) {
            const int kk = x / D, c = x % D;
            const int64_t j = kid[kk];
            float kv = 0.f, vv = 0.f;
            if (j >= 0) {
                const int64_t row = (int64_t)b * a.Nmax + j;
                kv = load_elem(a.k, a.kv_dtype, row * D + c);
                vv = load_elem(a.v, a.kv_dtype, row * D + c);
                if (a.kv_dtype == HS2_FP8_E4M3) { kv *= a.k_scale[row]; vv *= a.v_scale[row]; }
            }
            ks[kk][c] = kv;
            vs[kk][c] = vv;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kGenTile / 8; ++u) {
            const int kk = (tid & 7) + 8 * u;
            float acc = 0.f;
#pragma unroll 8
            for (int c = 0; c < D; ++c) acc += qs[hh][c] * ks[kk][c];
            ss[hh][kk] = kid[kk] >= 0 ? acc : kNegInf;
        }
        __syncthreads();
        if (tid < 32) {
            float mt = kNegInf;
            for (int kk = 0; kk < kGenTile; ++kk) mt = fmaxf(mt, ss[tid][kk]);
            const float mo = m_s[tid], mn = fmaxf(mo, mt);
            al_s[tid] = (mn == kNegInf) ? 1.f : exp2f(mo - mn);
            m_s[tid] = mn;
        }
        __syncthreads();
        for (int x = tid; x < 32 * kGenTile; x += kGenThreads) {
            const int h = x / kGenTile, kk = x % kGenTile;
            const float sv = ss[h][kk];
            ss[h][kk] = (sv == kNegInf) ? 0.f : exp2f(sv - m_s[h]);
        }
        __syncthreads();
        if (tid < 32) {
            float sum = 0.f;
            for (int kk = 0; kk < kGenTile; ++kk) sum += ss[tid][kk];
            l_s[tid] = l_s[tid] * al_s[tid] + sum;
        }
        const float al = al_s[hh];
#pragma unroll
        for (int u = 0; u < NO; ++u) {
            const int dv = dv0 + 8 * u;
            float acc = oacc[u] * al;
            for (int kk = 0; kk < kGenTile; ++kk) acc += ss[hh][kk] * vs[kk][dv];
            oacc[u] = acc;
        }
    }
    __syncthreads();
    if (hh < H) {
        if (a.part) {
            float* p = a.part + (((int64_t)r * a.nsplit + split) * H + hh) * (D + 2);
#pragma unroll
            for (int u = 0; u < NO; ++u) p[dv0 + 8 * u] = oacc[u];
            if (dv0 == 0) { p[D] = m_s[hh]; p[D + 1] = l_s[hh]; }
        } else {
            // single split: the workgroup saw every key of the row, normalise in place
            const float l = l_s[hh];
            float* po = a.o + ((int64_t)r * H + hh) * D;
#pragma unroll
            for (int u = 0; u < NO; ++u) po[dv0 + 8 * u] = l > 0.f ? oacc[u] / l : 0.f;
            if (dv0 == 0 && a.lse) a.lse[(int64_t)r * H + hh] = l > 0.f ? m_s[hh] + log2f(l) : kNegInf;
        }
    }
}

// Merge the splits of each row: m = max m_c, l = sum l_c 2^(m_c - m), o = sum o_c 2^(m_c - m) / l.
// A row with no visible key gets o = 0 and lse = -inf.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
    const int r = blockIdx.x;
    const int H = a.H, D = a.d, ns = a.nsplit;
    const float* base = a.part + (int64_t)r * ns * H * (D + 2);
    for (int x = threadIdx.x; x < H * D; x += blockDim.x) {
        const int h = x / D, c = x % D;
        float m = kNegInf;
        for (int s = 0; s < ns; ++s) m = fmaxf(m, base[((int64_t)s * H + h) * (D + 2) + D]);
        float l = 0.f, o = 0.f;
        if (m != kNegInf) {
            for (int s = 0; s < ns; ++s) {
                const float* p = base + ((int64_t)s * H + h) * (D + 2);
                const float ms = p[D];
                if (ms == kNegInf) continue;
                const float w = exp2f(ms - m);
                l += p[D + 1] * w;
                o += p[c] * w;
            }
        }
        a.o[((int64_t)r * H + h) * D + c] = l > 0.f ? o / l : 0.f;
        if (c == 0 && a.lse) a.lse[(int64_t)r * H + h] = l > 0.f ? m + log2f(l) : kNegInf;
    }
}

// Selection score of every candidate key j in [0, t - window]:
//   score(j) = sum_h 2^(x_h(j) - lse_h),  lse_h = m_h + log2 l_h from the full layer,
// i.e. the sum over heads of the full layer's softmax probabilities.  Optionally adds the
// top radix digit of each score to the row histogram used by the select kernels.
template <int D>
__global__ __launch_bounds__(kGenThreads) void score_generic_kernel(ScoreArgs a) {
    __shared__ float qs[32][D];
    __shared__ float ks[kGenTile][D + 1];
    __shared__ float ss[32][kGenTile + 1];
    __shared__ float lse_s[32];
    __shared__ uint32_t hist[kHistBins];

    const int r = blockIdx.x, split = blockIdx.y, tid = threadIdx.x;
    const int b = r / a.Tq;
    const int H = a.H;
    const int64_t t = row_pos(a.q_pos, a.kv_len, r, a.Tq, a.Nmax);
    const int64_t C = cand_count(t, a.window);
    const int64_t e0 = (int64_t)split * a.chunk;
    const int64_t e1 = e0 + a.chunk < C ? e0 + a.chunk : C;
    if (e0 >= e1) return;

    for (int x = tid; x < 32 * D; x += kGenThreads) {
        const int h = x / D, c = x % D;
        qs[h][c] = h < H ? load_elem(a.q, a.q_dtype, ((int64_t)r * H + h) * D + c) * a.scale_log2 : 0.f;
    }
    if (tid < 32) lse_s[tid] = tid < H ? a.lse[(int64_t)r * H + tid] : 0.f;
    if (a.rowhist)
        for (int x = tid; x < kHistBins; x += kGenThreads) hist[x] = 0;
    const int hh = tid >> 3;

    for (int64_t eb = e0; eb < e1; eb += kGenTile) {
        __syncthreads();
        for (int x = tid; x < kGenTile * D; x += kGenThreads) {
            const int kk = x / D, c = x % D;
            const int64_t j = eb + kk;
            float kv = 0.f;
            if (j < e1) {
                const int64_t row = (int64_t)b * a.Nmax + j;
                kv = load_elem(a.k, a.kv_dtype, row * D + c);
                if (a.kv_dtype == HS2_FP8_E4M3) kv *= a.k_scale[row];
            }
            ks[kk][c] = kv;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kGenTile / 8; ++u) {
            const int kk = (tid & 7) + 8 * u;
            float acc = 0.f;
#pragma unroll 8
            for (int c = 0; c < D; ++c) acc += qs[hh][c] * ks[kk][c];
            ss[hh][kk] = acc;
        }
        __syncthreads();
        if (tid < kGenTile) {
            const int64_t j = eb + tid;
            if (j < e1) {
                float sc = 0.f;
                for (int h = 0; h < H; ++h) sc += exp2f(ss[h][tid] - lse_s[h]);
                a.scores[(int64_t)r * a.cstride + j] = sc;
                if (a.rowhist) atomicAdd(&hist[__float_as_uint(sc) >> 21], 1u);
            }
        }
    }
    if (a.rowhist) {
        __syncthreads();
        for (int x = tid; x < kHistBins; x += kGenThreads)
            if (hist[x]) atomicAdd(&a.rowhist[(int64_t)r * kHistBins + x], hist[x]);
    }
}

hipError_t launch_attn_generic(const AttnArgs& a, const char* name, hipStream_t s) {
    ProfScope ps(name, s);
    dim3 grid(a.B * a.Tq, a.nsplit);
    if (a.d == 64) attn_generic_kernel<64><<<grid, kGenThreads, 0, s>>>(a);
    else attn_generic_kernel<128><<<grid, kGenThreads, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs& a, const char* name, hipStream_t s) {
    ProfScope ps(name, s);
    attn_combine_kernel<<<a.B * a.Tq, 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_score_generic(const ScoreArgs& a, hipStream_t s) {
    ProfScope ps("score_generic", s);
    dim3 grid(a.B * a.Tq, a.nsplit);
    if (a.d == 64) score_generic_kernel<64><<<grid, kGenThreads, 0, s>>>(a);
    else score_generic_kernel<128><<<grid, kGenThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace hs2
