// Merge of the key splits of the row attention kernel: o = sum_s 2^(m_s - M) o_s / L with
// M = max_s m_s and L = sum_s 2^(m_s - M) l_s per (row, head), from the MFMA partial layout
// part [R, nsplit, H, d] (unnormalised o) and part_ml [R, nsplit, H, 2] (m, l; base 2).
#pragma once

#include "hs2_device.h"

#include <type_traits>

namespace hs2 {

constexpr int kCombineNarrowMax = 32;  // splits up to which a (row, head) workgroup merges alone

// The row of a workgroup and its buffers (multi-layer launches: block row x is row x % R of
// layer x / R).
struct CombineRow {
    int r;
    const float* part;
    const float* part_ml;
    float* o;
    float* lse;
};
__device__ __forceinline__ CombineRow combine_row(const AttnArgs& a, int bx) {
    CombineRow c{bx, a.part, a.part_ml, a.o, a.lse};
    if (a.nlayer > 1) {
        const int R = a.B * a.Tq, layer = c.r / R;
        c.r -= layer * R;
        c.part += layer * a.part_lstride;
        c.part_ml += layer * a.ml_lstride;
        c.o = a.ol[layer];
        c.lse = nullptr;
    }
    return c;
}

// ---- merge of the splits of each row ----------------------------------------------------------------
// Many splits (long rows): grid (row, head, D/16), 256 threads = 16 dims x 16 split lanes.  Every
// workgroup first reduces the per-split maxima and sums of its head (tiny), then sums its 16
// dims over the splits.
struct CombineWideLds {
    float red[16][17];
    float wred[4];
};

// One workgroup of 256 threads: block row bx, head h, dims 16 bz .. 16 bz + 15.  SK (m, l) pairs
// per thread and the first U0 splits per output dim are loaded up front (sized to the split count,
// so that no load is a clamped repeat).
template <int D, int SK, int U0>
__device__ __forceinline__ void combine_wide_impl(const AttnArgs& a, int bx, int h, int bz, CombineWideLds& S) {
    float (&red)[16][17] = S.red;
    float (&wred)[4] = S.wred;
    const CombineRow cr = combine_row(a, bx);
    const int r = cr.r, H = a.H, ns = a.nsplit;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    // split s: o at obase + s * ostride, (m, l) at mbase + s * mstride
    const float* obase = cr.part + ((int64_t)r * ns * H + h) * D;
    const float* mbase = cr.part_ml + ((int64_t)r * ns * H + h) * 2;
    const int64_t ostride = (int64_t)H * D, mstride = (int64_t)H * 2;
    const int dl = tid & 15, sl = tid >> 4;
    const int dv = bz * 16 + dl;
    // Every load that does not depend on the maximum is issued before the first reduction: the
    // (m, l) pairs of this thread's splits tid + 256 k and the first U0 splits sl + 16 u of its
    // output dim (loads are clamped to the last split and masked where used), so up to 256 splits
    // cost one round trip instead of three.
    float2 st[SK];
#pragma unroll
    for (int k = 0; k < SK; ++k) {
        const int s = tid + 256 * k;
        st[k] = *(const float2*)(mbase + (int64_t)(s < ns ? s : ns - 1) * mstride);
    }
    float mu0[U0], ou0[U0];
#pragma unroll
    for (int u = 0; u < U0; ++u) {
        const int s = sl + 16 * u < ns ? sl + 16 * u : ns - 1;
        mu0[u] = mbase[s * mstride];
        ou0[u] = obase[s * ostride + dv];
    }
    float m = kNegInf;
    for (int k = 0; k < SK; ++k)
        if (tid + 256 * k < ns) m = fmaxf(m, st[k].x);
    for (int s = tid + 256 * SK; s < ns; s += 256) m = fmaxf(m, mbase[s * mstride]);
    m = wave_max(m);
    if (lane == 0) wred[wv] = m;
    __syncthreads();
    const float M = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
    __syncthreads();
    float l = 0.f;
    if (M != kNegInf) {
#pragma unroll
        for (int k = 0; k < SK; ++k)
            if (tid + 256 * k < ns && st[k].x != kNegInf) l += st[k].y * exp2f(st[k].x - M);
        for (int s = tid + 256 * SK; s < ns; s += 256) {
            const float ms = mbase[s * mstride];
            l += ms == kNegInf ? 0.f : mbase[s * mstride + 1] * exp2f(ms - M);
        }
    }
    l = wave_sum(l);
    if (lane == 0) wred[wv] = l;
    __syncthreads();
    const float Ltot = wred[0] + wred[1] + wred[2] + wred[3];
    float acc = 0.f;
    if (M != kNegInf) {
        {
            float part = 0.f;
#pragma unroll
            for (int u = 0; u < U0; ++u)
                part += (sl + 16 * u < ns && mu0[u] != kNegInf) ? ou0[u] * exp2f(mu0[u] - M) : 0.f;
            acc += part;
        }
        // the remaining splits in batches of U per thread with all their loads in flight together
        // (16, then 8), so a long row's merge takes a few round trips instead of one per four splits
        int s = sl + 16 * U0;
        auto batch = [&](auto u_c) {
            constexpr int U = decltype(u_c)::value;
            for (; s + 16 * (U - 1) < ns; s += 16 * U) {
                float mu[U], ou[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    mu[u] = mbase[(s + 16 * u) * mstride];
                    ou[u] = obase[(s + 16 * u) * ostride + dv];
                }
                float part = 0.f;
#pragma unroll
                for (int u = 0; u < U; ++u) part += mu[u] == kNegInf ? 0.f : ou[u] * exp2f(mu[u] - M);
                acc += part;
            }
        };
        batch(std::integral_constant<int, 16>{});
        batch(std::integral_constant<int, 8>{});
        for (; s < ns; s += 16) {
            const float ms = mbase[s * mstride];
            if (ms != kNegInf) acc += obase[s * ostride + dv] * exp2f(ms - M);
        }
    }
    red[sl][dl] = acc;
    __syncthreads();
    if (tid < 16) {
        float tot = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) tot += red[q][tid];
        const int dvo = bz * 16 + tid;
        cr.o[((int64_t)r * H + h) * D + dvo] = Ltot > 0.f ? tot / Ltot : 0.f;
        if (dvo == 0 && cr.lse) cr.lse[(int64_t)r * H + h] = Ltot > 0.f ? M + log2f(Ltot) : kNegInf;
    }
}

template <int D>
__device__ __forceinline__ void combine_wide_body(const AttnArgs& a, int bx, int h, int bz, CombineWideLds& S) {
    if (a.nsplit <= 128) combine_wide_impl<D, 1, 8>(a, bx, h, bz, S);
    else if (a.nsplit <= 256) combine_wide_impl<D, 1, 16>(a, bx, h, bz, S);
    else if (a.nsplit <= 512) combine_wide_impl<D, 2, 16>(a, bx, h, bz, S);
    else combine_wide_impl<D, 4, 16>(a, bx, h, bz, S);
}

// Few splits: one workgroup per (row, head), one thread per dv.  Splits are merged in batches of 16 whose
// loads are all in flight together, with the running maximum rescaled between batches; the
// (m, l) loads of a batch are the same for every thread of the workgroup.
// Threads 0 .. D-1 of a workgroup: block row bx, head h (no barriers, so extra threads may skip it).
template <int D>
__device__ __forceinline__ void combine_narrow_body(const AttnArgs& a, int bx, int h) {
    constexpr int BATCH = 16;
    const CombineRow cr = combine_row(a, bx);
    const int r = cr.r, H = a.H, ns = a.nsplit;
    const int dv = threadIdx.x;
    const float* obase = cr.part + ((int64_t)r * ns * H + h) * D + dv;     // split s at + s * H * D
    const float* mbase = cr.part_ml + ((int64_t)r * ns * H + h) * 2;      // split s at + s * H * 2
    float M = kNegInf, L = 0.f, acc = 0.f;
    for (int s0 = 0; s0 < ns; s0 += BATCH) {
        float2 ml[BATCH];
        float ov[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int sp = s0 + u < ns ? s0 + u : ns - 1;
            ml[u] = *(const float2*)(mbase + (int64_t)sp * H * 2);
            ov[u] = obase[(int64_t)sp * H * D];
        }
        float mb = kNegInf;
#pragma unroll
        for (int u = 0; u < BATCH; ++u) if (s0 + u < ns) mb = fmaxf(mb, ml[u].x);
        const float Mn = fmaxf(M, mb);
        if (Mn == kNegInf) continue;                 // nothing seen yet
        const float c = M == kNegInf ? 0.f : exp2f(M - Mn);
        L *= c;
        acc *= c;
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            if (s0 + u < ns && ml[u].x != kNegInf) {
                const float wgt = exp2f(ml[u].x - Mn);
                L += ml[u].y * wgt;
                acc += ov[u] * wgt;
            }
        }
        M = Mn;
    }
    cr.o[((int64_t)r * H + h) * D + dv] = L > 0.f ? acc / L : 0.f;
    if (dv == 0 && cr.lse) cr.lse[(int64_t)r * H + h] = L > 0.f ? M + log2f(L) : kNegInf;
}

}  // namespace hs2
