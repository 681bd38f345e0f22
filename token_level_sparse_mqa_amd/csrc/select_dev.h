// Token-level top-k selection with a forced recent window: device code.
//
// Per query row at position t (kucoin news flash; lynxflow blog, "Token-Level Sparse
// Selection"): the k_global best candidates j in [0, t - window] by (score desc, index asc),
// written ascending, then -1 padding; followed by the window max(0, t-window+1)..t and -1
// padding.  Scores are sums of probabilities, hence >= 0, so their binary32 bit patterns
// order like the values and an exact radix select over the 32 bits finds the k-th largest
// score T.  Everything above T is picked; among scores equal to T the lowest indices are
// picked.  All decisions are taken on the bit patterns: integer work, bit-exact.
//
// Kernels (radix digits [31:21] [20:10] [9:0]):
//   select_hist    per row segment: histogram of the top digit, summed into a row histogram
//   select_digit   per row (launches of many rows): the k-th's top digit and the count above
//                  it, found once instead of in every workgroup of the next two kernels
//   select_gather  per row segment: entries whose top digit is above the k-th's are sure
//                  picks; entries in the k-th's bucket become candidates (value, index)
//   select_finish  per row: resolves the remaining digits and the ties among the candidates
//                  in LDS, sorts the k picks ascending, writes the window and padding.  When
//                  the k-th bucket holds more than kSelCap entries it falls back to exact
//                  streaming passes over the row in global memory.
#pragma once

#include "hs2_device.h"

namespace hs2 {

__device__ __forceinline__ uint32_t dig1(uint32_t key) { return key >> 21; }
__device__ __forceinline__ uint32_t dig2(uint32_t key) { return (key >> 10) & 0x7ffu; }
__device__ __forceinline__ uint32_t dig3(uint32_t key) { return key & 0x3ffu; }

// Given a histogram over NBINS digits (global or LDS memory) and a rank k, find the digit
// holding the k-th largest entry and the number of entries with a larger digit.  Every wave
// that calls it computes the same result on its own (no barrier): lane l sums the NBINS/64
// digits NBINS-1-l*PER .. NBINS-(l+1)*PER, a shuffle scan over the lanes gives each lane the
// count above its digits, and the lane that holds the k-th entry broadcasts it.  Should the
// histogram hold fewer than k entries, digit 0 is reported (callers bound their writes).
// Split in two so that callers can issue the histogram loads early: wave_load_hist reads this
// lane's NBINS/64 digits, wave_digit_from searches them.
template <int NBINS>
__device__ __forceinline__ void wave_load_hist(const uint32_t* hist, uint32_t (&c)[NBINS / 64]) {
    constexpr int PER = NBINS / 64;
    const int lane = threadIdx.x & 63;
    const uint32_t* hb = hist + NBINS - (lane + 1) * PER;   // this lane's digits, ascending
#pragma unroll
    for (int i = 0; i < PER; i += 4) {
        const uint4 q = *(const uint4*)(hb + i);
        c[i] = q.x; c[i + 1] = q.y; c[i + 2] = q.z; c[i + 3] = q.w;
    }
}

template <int NBINS>
__device__ __forceinline__ void wave_digit_from(const uint32_t (&c)[NBINS / 64], uint32_t k, uint32_t& digit,
                                                uint32_t& above) {
    constexpr int PER = NBINS / 64;
    const int lane = threadIdx.x & 63;
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) local += c[i];
    const uint32_t incl = wave_incl_scan(local);
    const uint32_t total = lane_value(incl, 63);
    uint32_t run = incl - local;        // entries with a digit above this lane's digits
    int found = -1;
    uint32_t fab = 0;
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {   // this lane's digits, descending
        if (run < k && run + c[i] >= k) { found = NBINS - (lane + 1) * PER + i; fab = run; }
        run += c[i];
    }
    const uint64_t m = __ballot(found >= 0);
    if (m) {
        const int src = __ffsll((unsigned long long)m) - 1;
        digit = lane_value((uint32_t)found, src);
        above = lane_value(fab, src);
    } else {
        digit = 0;
        above = total - lane_value(c[0], 63);    // lane 63 holds digits PER-1 .. 0
    }
}

template <int NBINS>
__device__ __forceinline__ void wave_find_digit(const uint32_t* hist, uint32_t k, uint32_t& digit, uint32_t& above) {
    uint32_t c[NBINS / 64];
    wave_load_hist<NBINS>(hist, c);
    wave_digit_from<NBINS>(c, k, digit, above);
}

// Block-level digit search for a histogram in LDS: thread t reads consecutive digits (no bank
// conflicts) and a block scan orders the threads.  Same result convention as wave_find_digit;
// every thread of the block calls it and receives the result.
template <int NT>
__device__ void block_find_digit(const uint32_t* hist, int nbins, uint32_t k, uint32_t& digit, uint32_t& above,
                                 uint32_t* tmp, uint32_t* res) {
    const int per = (nbins + NT - 1) / NT;
    const int x0 = threadIdx.x * per;
    uint32_t local = 0;
    for (int x = x0; x < x0 + per && x < nbins; ++x) local += hist[nbins - 1 - x];
    uint32_t total;
    uint32_t run = block_excl_scan<NT>(local, tmp, &total);
    for (int x = x0; x < x0 + per && x < nbins; ++x) {
        const uint32_t c = hist[nbins - 1 - x];
        const bool last = x == nbins - 1;
        if ((run < k && run + c >= k) || (last && run + c < k)) { res[0] = (uint32_t)(nbins - 1 - x); res[1] = run; }
        run += c;
    }
    __syncthreads();
    digit = res[0];
    above = res[1];
}

__device__ __forceinline__ void row_info(const SelectArgs& a, int r, int64_t* t, int64_t* C) {
    *t = row_pos(a.q_pos, a.kv_len, r, a.Tq, a.Nmax);
    *C = cand_count(*t, a.window);
}

// Wave-aggregated append: returns the slot of this lane (valid where `pred`).
__device__ __forceinline__ uint32_t wave_append(uint32_t* counter, bool pred) {
    const uint64_t m = __ballot(pred);
    if (!m) return 0;
    const int lane = threadIdx.x & 63;
    const int leader = __ffsll((unsigned long long)m) - 1;
    uint32_t base = 0;
    if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(m));
    base = lane_value(base, leader);
    return base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
}

// One workgroup of 256 threads: row r, segment seg of kSelSeg positions.  The counts of sure
// picks (high half) and bucket candidates (low half; at most 4096 each per workgroup) are packed
// into one word: a wave scan of the lanes' words, then one thread adds the four wave totals and
// reserves space in both row lists with a single 64-bit atomic (counter 0 in the low word,
// counter 1 in the high word; one atomic per workgroup, since atomics on a row's counters
// serialise).  The order of the entries in the lists is arbitrary; the finish sorts what it
// keeps.
struct GatherLds {
    uint32_t wtot[4];
    uint32_t wbase[4][2];
};

// GIVEN: the row's digit comes from a.digits (written by select_digit_kernel) instead of a search
// over the row histogram in every wave; otherwise the waves search it and the first segment's
// workgroup writes it to a.digits for the finish.
template <bool GIVEN = false>
__device__ __forceinline__ void select_gather_body(const SelectArgs& a, int r, int seg, GatherLds& S) {
    constexpr int PER = kSelSeg / 256;
    // the segment's scores (every position below Nmax is inside the row's buffer; those past the
    // candidate count are masked below) and the row histogram or digit are loaded together with
    // the row's position: one memory round trip before the classification
    const int64_t j0 = (int64_t)seg * kSelSeg;
    const float* sc = a.scores + (int64_t)r * a.cstride;
    uint32_t key[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int64_t j = j0 + u * 256 + threadIdx.x;
        key[u] = j < a.Nmax ? __float_as_uint(sc[j]) : 0u;
    }
    uint32_t hc[kHistBins / 64];
    uint32_t b1 = 0, above1;
    if constexpr (GIVEN) b1 = a.digits[2 * (int64_t)r];
    else wave_load_hist<kHistBins>(a.rowhist + (int64_t)r * kHistBins, hc);
    int64_t t, C;
    row_info(a, r, &t, &C);
    if (C <= a.k_global) return;
    if (j0 >= C) return;
    const int64_t j1 = j0 + kSelSeg < C ? j0 + kSelSeg : C;
    if constexpr (!GIVEN) {
        wave_digit_from<kHistBins>(hc, (uint32_t)a.k_global, b1, above1);
        // the first segment's workgroup records the digit, so the finish needs no search of its own
        if (seg == 0 && threadIdx.x == 0 && a.digits) {
            a.digits[2 * (int64_t)r] = b1;
            a.digits[2 * (int64_t)r + 1] = above1;
        }
    }
    // bit u of sm / cm: entry u is a sure pick / a bucket candidate (kept in vector registers, so
    // the sixteen per-entry conditions need no lane masks across the reservation below)
    const int nvalid = (int)(j1 - j0);
    uint32_t sm = 0, cm = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const bool valid = u * 256 + (int)threadIdx.x < nvalid;
        const uint32_t dg = dig1(key[u]);
        sm |= (valid && dg > b1) ? (1u << u) : 0u;
        cm |= (valid && dg == b1) ? (1u << u) : 0u;
    }
    const uint32_t ns = (uint32_t)__popc(sm), nc = (uint32_t)__popc(cm);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint32_t mine = (ns << 16) | nc;
    const uint32_t incl = wave_incl_scan(mine);
    if (lane == 63) S.wtot[w] = incl;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t run = 0;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const uint32_t tw = S.wtot[x];
            S.wbase[x][0] = run >> 16;
            S.wbase[x][1] = run & 0xffffu;
            run += tw;
        }
        unsigned long long old = 0;
        if (run)
            old = atomicAdd((unsigned long long*)(a.counters + (int64_t)r * 4),
                            ((unsigned long long)(run & 0xffffu) << 32) | (run >> 16));
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            S.wbase[x][0] += (uint32_t)old;
            S.wbase[x][1] += (uint32_t)(old >> 32);
        }
    }
    __syncthreads();
    const uint32_t excl = incl - mine;
    uint32_t ps = S.wbase[w][0] + (excl >> 16);
    uint32_t pc = S.wbase[w][1] + (excl & 0xffffu);
    int32_t* sure = a.sure + (int64_t)r * a.k_global;
    uint2* cand = a.cand + (int64_t)r * kSelCap;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int32_t j = (int32_t)(j0 + u * 256 + threadIdx.x);
        if ((sm >> u) & 1u) {
            // fewer than k_global entries lie above the k-th's bucket; the bound only matters
            // if the row histogram disagreed with the scores
            if (ps < (uint32_t)a.k_global) sure[ps] = j;
            ++ps;
        } else if ((cm >> u) & 1u) {
            if (pc < (uint32_t)kSelCap) cand[pc] = make_uint2(key[u], (uint32_t)j);
            ++pc;
        }
    }
}

constexpr int kFinThreads = 1024;     // threads of the standalone finish kernel

// Ascending bitonic sort of n (power of two) 32-bit values in LDS.
template <int NT>
__device__ void bitonic_sort_i32(int32_t* v, int n) {
    for (int k = 2; k <= n; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < n; i += NT) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const int32_t x = v[i], y = v[ixj];
                    const bool up = (i & k) == 0;
                    if ((x > y) == up) { v[i] = y; v[ixj] = x; }
                }
            }
            __syncthreads();
        }
    }
}

// Writes the K <= NT distinct picks out[0..K) (values in [0, C)) to irow in ascending
// order.  Each pick goes to bucket v >> sh (at most kRankBuckets buckets cover [0, C)); a scan
// of the bucket counts gives each bucket's first output position, and a pick's rank within its
// bucket is the number of smaller picks there (buckets span 2^sh indices, so they hold few
// picks unless the picks cluster).  cnt and start hold kRankBuckets entries, items K.
constexpr int kRankBuckets = 4096;

template <int NT>
__device__ void rank_sort_picks(const int32_t* out, int K, int64_t C, int32_t* irow, uint32_t* cnt,
                                uint32_t* start, int32_t* items, uint32_t* tmp) {
    int sh = 0;
    while (((C - 1) >> sh) >= kRankBuckets) ++sh;
    for (int x = threadIdx.x; x < kRankBuckets; x += NT) cnt[x] = 0;
    __syncthreads();
    const int t = threadIdx.x;
    const int32_t v = t < K ? out[t] : -1;
    const bool mine = v >= 0 && (int64_t)v < C;     // always, unless the counts disagreed
    const int b = mine ? (int)((int64_t)v >> sh) : 0;
    uint32_t slot = 0;
    if (mine) slot = atomicAdd(&cnt[b], 1u);
    __syncthreads();
    constexpr int PER = kRankBuckets / NT;
    uint32_t c[PER];
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) { c[i] = cnt[PER * t + i]; sum += c[i]; }
    uint32_t total;
    uint32_t base = block_excl_scan<NT>(sum, tmp, &total);
#pragma unroll
    for (int i = 0; i < PER; ++i) { start[PER * t + i] = base; base += c[i]; }
    __syncthreads();
    if (mine) items[start[b] + slot] = v;
    __syncthreads();
    if (mine) {
        const uint32_t s0 = start[b], n = cnt[b];
        uint32_t rank = s0;
        for (uint32_t i = 0; i < n; ++i) rank += items[s0 + i] < v ? 1u : 0u;
        irow[rank] = v;
    }
}

template <int NT>
struct FinishLds {
    __attribute__((aligned(16))) uint32_t hist[kHistBins];
    uint32_t ckey[kSelCap];
    int32_t cidx[kSelCap];
    int32_t out[4096];
    uint32_t tmp[NT / 64 + 1];
    uint32_t res[2];
    uint32_t lcount[2];
};

// One workgroup of NT threads: row r.
template <int NT, bool GIVEN = false>
__device__ __forceinline__ void select_finish_body(const SelectArgs& a, int r, FinishLds<NT>& S) {
    uint32_t (&hist)[kHistBins] = S.hist;
    uint32_t (&ckey)[kSelCap] = S.ckey;
    int32_t (&cidx)[kSelCap] = S.cidx;
    int32_t (&out)[4096] = S.out;
    uint32_t (&tmp)[NT / 64 + 1] = S.tmp;
    uint32_t (&res)[2] = S.res;
    uint32_t (&lcount)[2] = S.lcount;

    const int K = a.k_global, W = a.window;
    // Every global load of the row is issued before any is used, so together they cost one memory
    // round trip: the candidate slots, the candidate count, the sure list, the row histogram (or
    // the row's digit) and the row's position.  All lie at fixed, in-bounds addresses; slots past
    // the counts hold stale values that are never used.
    constexpr int CU = kSelCap / NT;
    const uint2* cg = a.cand + (int64_t)r * kSelCap;
    uint2 cpre[CU];
#pragma unroll
    for (int u = 0; u < CU; ++u) cpre[u] = cg[threadIdx.x + u * NT];
    const uint32_t n_cand = a.counters[(int64_t)r * 4 + 1];
    constexpr int SU = (4096 + NT - 1) / NT;       // sure slots per thread (k_global <= 4096)
    int32_t spre[SU];
#pragma unroll
    for (int u = 0; u < SU; ++u) {
        const int x = threadIdx.x + u * NT;
        spre[u] = a.sure[(int64_t)r * K + (x < K ? x : K - 1)];
    }
    constexpr int HU = kHistBins / NT;
    uint32_t hpre[HU];
    uint32_t b1 = 0, above1 = 0;
    if constexpr (GIVEN) {
        b1 = a.digits[2 * (int64_t)r];
        above1 = a.digits[2 * (int64_t)r + 1];
    } else {
#pragma unroll
        for (int u = 0; u < HU; ++u) hpre[u] = a.rowhist[(int64_t)r * kHistBins + threadIdx.x + u * NT];
    }
    int64_t t, C;
    row_info(a, r, &t, &C);
    int32_t* irow = a.idx + (int64_t)r * (K + W);
    const float* sc = a.scores + (int64_t)r * a.cstride;

    // window segment and the optional score dump
    for (int w = threadIdx.x; w < W; w += NT) {
        int32_t v = -1;
        if (t >= 0) {
            const int64_t first = t - W + 1 > 0 ? t - W + 1 : 0;
            const int64_t jj = first + w;
            v = jj <= t ? (int32_t)jj : -1;
        }
        irow[K + w] = v;
    }
    if (a.scores_dbg) {
        float* dbg = a.scores_dbg + (int64_t)r * a.Nmax;
        for (int64_t j = threadIdx.x; j < a.Nmax; j += NT) dbg[j] = j < C ? sc[j] : -1.0f;
    }
    if (C <= K) {
        for (int j = threadIdx.x; j < K; j += NT) irow[j] = j < C ? j : -1;
        return;
    }
    if constexpr (!GIVEN) {
        // the k-th's top digit from the row histogram, staged in LDS (the block search ends with a
        // barrier, after which the histogram space is free for the next digits)
#pragma unroll
        for (int u = 0; u < HU; ++u) hist[threadIdx.x + u * NT] = hpre[u];
        __syncthreads();
        block_find_digit<NT>(hist, kHistBins, (uint32_t)K, b1, above1, tmp, res);
    }
    const uint32_t k1 = (uint32_t)K - above1;
    uint32_t b2, b3, above2, above3;

    if (n_cand <= (uint32_t)kSelCap) {
        // ---- fast path: the k-th bucket is in LDS ----
#pragma unroll
        for (int u = 0; u < CU; ++u) {
            const uint32_t x = threadIdx.x + u * NT;
            if (x < n_cand) { ckey[x] = cpre[u].x; cidx[x] = (int32_t)cpre[u].y; }
        }
        for (int x = threadIdx.x; x < kHistBins; x += NT) hist[x] = 0;
        __syncthreads();
        for (uint32_t x = threadIdx.x; x < n_cand; x += NT) atomicAdd(&hist[dig2(ckey[x])], 1u);
        __syncthreads();
        block_find_digit<NT>(hist, kHistBins, k1, b2, above2, tmp, res);
        const uint32_t k2 = k1 - above2;
        for (int x = threadIdx.x; x < kHistBins; x += NT) hist[x] = 0;
        __syncthreads();
        for (uint32_t x = threadIdx.x; x < n_cand; x += NT)
            if (dig2(ckey[x]) == b2) atomicAdd(&hist[dig3(ckey[x])], 1u);
        __syncthreads();
        block_find_digit<NT>(hist, 1024, k2, b3, above3, tmp, res);
        const uint32_t need_eq = k2 - above3;          // ties at T still needed
        const uint32_t n_eq = hist[b3];
        const uint32_t T = (b1 << 21) | (b2 << 10) | b3;
        // sure picks from the gather pass
        const uint32_t n_sure = above1 < (uint32_t)K ? above1 : (uint32_t)K;
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            const uint32_t x = threadIdx.x + u * NT;
            if (x < n_sure) out[x] = spre[u];
        }
        if (threadIdx.x == 0) { lcount[0] = n_sure; lcount[1] = 0; }
        // classify the bucket: above T -> picked; equal to T -> tie list (reusing ckey storage)
        uint32_t myk[kSelCap / NT];
        int32_t myi[kSelCap / NT];
#pragma unroll
        for (int u = 0; u < kSelCap / NT; ++u) {
            const uint32_t x = threadIdx.x + u * NT;
            myk[u] = x < n_cand ? ckey[x] : 0u;
            myi[u] = x < n_cand ? cidx[x] : -1;
        }
        __syncthreads();
        int32_t* ties = (int32_t*)ckey;
#pragma unroll
        for (int u = 0; u < kSelCap / NT; ++u) {
            const uint32_t x = threadIdx.x + u * NT;
            if (x < n_cand) {
                if (myk[u] > T) {
                    const uint32_t o = atomicAdd(&lcount[0], 1u);
                    if (o < (uint32_t)K) out[o] = myi[u];
                } else if (myk[u] == T) {
                    ties[atomicAdd(&lcount[1], 1u)] = myi[u];   // at most n_cand <= kSelCap
                }
            }
        }
        __syncthreads();
        const uint32_t base = lcount[0];
        if (need_eq == n_eq) {
            for (uint32_t x = threadIdx.x; x < n_eq; x += NT)
                if (base + x < (uint32_t)K) out[base + x] = ties[x];
        } else {
            int np = 1;
            while (np < (int)n_eq) np <<= 1;
            for (int x = threadIdx.x; x < np; x += NT) if (x >= (int)n_eq) ties[x] = 0x7fffffff;
            __syncthreads();
            bitonic_sort_i32<NT>(ties, np);
            for (uint32_t x = threadIdx.x; x < need_eq && x < n_eq; x += NT)
                if (base + x < (uint32_t)K) out[base + x] = ties[x];
        }
        __syncthreads();
        if (K <= NT) {
            // the candidate and histogram arrays are free now
            rank_sort_picks<NT>(out, K, C, irow, ckey, (uint32_t*)cidx, (int32_t*)hist, tmp);
        } else {
            int np = 1;
            while (np < K) np <<= 1;
            for (int x = threadIdx.x; x < np; x += NT) if (x >= K) out[x] = 0x7fffffff;
            __syncthreads();
            bitonic_sort_i32<NT>(out, np);
            for (int x = threadIdx.x; x < K; x += NT) irow[x] = out[x];
        }
        return;
    }

    // ---- fallback: exact streaming passes over the row ----
    // This path serves buckets of more than kSelCap entries, typically long runs of equal scores:
    // a wave whose counted lanes all fall into one bin adds them with a single atomic.
    auto hist_add = [&](bool pred, uint32_t bin) {
        const uint64_t m = __ballot(pred);
        if (!m) return;
        const int lead = __ffsll((unsigned long long)m) - 1;
        const uint32_t lb = lane_value(bin, lead);
        if (__ballot(pred && bin != lb) == 0) {
            if ((int)(threadIdx.x & 63) == lead) atomicAdd(&hist[lb], (uint32_t)__popcll(m));
        } else if (pred) {
            atomicAdd(&hist[bin], 1u);
        }
    };
    // The row's scores are read UB positions per thread at a time, all of a batch's loads in flight
    // together (one memory round trip per NT * UB positions; eight per thread measured slower).
    constexpr int UB = 4;
    auto hist_pass = [&](auto count) {
        for (int64_t jb = 0; jb < C; jb += (int64_t)NT * UB) {
            uint32_t kk[UB];
#pragma unroll
            for (int u = 0; u < UB; ++u) {
                const int64_t j = jb + (int64_t)u * NT + threadIdx.x;
                kk[u] = j < C ? __float_as_uint(sc[j]) : 0u;
            }
#pragma unroll
            for (int u = 0; u < UB; ++u) count(jb + (int64_t)u * NT + threadIdx.x < C, kk[u]);
        }
    };
    for (int x = threadIdx.x; x < kHistBins; x += NT) hist[x] = 0;
    __syncthreads();
    hist_pass([&](bool valid, uint32_t key) { hist_add(valid && dig1(key) == b1, dig2(key)); });
    __syncthreads();
    block_find_digit<NT>(hist, kHistBins, k1, b2, above2, tmp, res);
    const uint32_t k2 = k1 - above2;
    const uint32_t pre = (b1 << 11) | b2;
    for (int x = threadIdx.x; x < kHistBins; x += NT) hist[x] = 0;
    __syncthreads();
    hist_pass([&](bool valid, uint32_t key) { hist_add(valid && (key >> 10) == pre, dig3(key)); });
    __syncthreads();
    block_find_digit<NT>(hist, 1024, k2, b3, above3, tmp, res);
    const uint32_t need_eq = k2 - above3;
    const uint32_t T = (b1 << 21) | (b2 << 10) | b3;
    // ordered pass: thread t takes the UB consecutive positions jb + UB t .. jb + UB t + UB - 1, so
    // thread order is position order; a block scan of the per-thread tie counts ranks the ties by
    // index, a second one places the picks
    uint32_t run_eq = 0, run_out = 0;
    for (int64_t jb = 0; jb < C; jb += (int64_t)NT * UB) {
        const int64_t jt = jb + (int64_t)threadIdx.x * UB;
        uint32_t kk[UB];
#pragma unroll
        for (int u = 0; u < UB; ++u) kk[u] = jt + u < C ? __float_as_uint(sc[jt + u]) : 0u;
        uint32_t neq = 0;
#pragma unroll
        for (int u = 0; u < UB; ++u) neq += (jt + u < C && kk[u] == T) ? 1u : 0u;
        uint32_t tot_eq;
        const uint32_t rank0 = run_eq + block_excl_scan<NT>(neq, tmp, &tot_eq);
        uint32_t npick = 0;
        {
            uint32_t rank = rank0;
#pragma unroll
            for (int u = 0; u < UB; ++u) {
                const bool valid = jt + u < C, eq = valid && kk[u] == T;
                npick += (valid && (kk[u] > T || (eq && rank < need_eq))) ? 1u : 0u;
                rank += eq ? 1u : 0u;
            }
        }
        uint32_t tot_pick;
        uint32_t pos = run_out + block_excl_scan<NT>(npick, tmp, &tot_pick);
        {
            uint32_t rank = rank0;
#pragma unroll
            for (int u = 0; u < UB; ++u) {
                const bool valid = jt + u < C, eq = valid && kk[u] == T;
                if (valid && (kk[u] > T || (eq && rank < need_eq))) {
                    if (pos < (uint32_t)K) irow[pos] = (int32_t)(jt + u);
                    ++pos;
                }
                rank += eq ? 1u : 0u;
            }
        }
        run_eq += tot_eq;
        run_out += tot_pick;
        // the picks number exactly K (everything above T and the lowest need_eq ties), so the
        // pass ends once they are placed (early, when ties at T hold the low indices)
        if (run_out >= (uint32_t)K) break;
    }
}

}  // namespace hs2
