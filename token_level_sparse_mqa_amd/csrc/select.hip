// Selection kernels.  Device code of the histogram digit search, the gather and the finish:
// select_dev.h (shared with the single-launch decode block).
#include "select_dev.h"

namespace hs2 {

__global__ __launch_bounds__(256) void select_hist_kernel(SelectArgs a) {
    __shared__ uint32_t hist[kHistBins];
    const int r = blockIdx.x, seg = blockIdx.y;
    int64_t t, C;
    row_info(a, r, &t, &C);
    if (C <= a.k_global) return;
    const int64_t j0 = (int64_t)seg * kSelSeg;
    if (j0 >= C) return;
    const int64_t j1 = j0 + kSelSeg < C ? j0 + kSelSeg : C;
    for (int x = threadIdx.x; x < kHistBins; x += 256) hist[x] = 0;
    __syncthreads();
    const float* sc = a.scores + (int64_t)r * a.cstride;
    for (int64_t j = j0 + threadIdx.x; j < j1; j += 256) atomicAdd(&hist[dig1(__float_as_uint(sc[j]))], 1u);
    __syncthreads();
    for (int x = threadIdx.x; x < kHistBins; x += 256)
        if (hist[x]) atomicAdd(&a.rowhist[(int64_t)r * kHistBins + x], hist[x]);
}

// One wave per row: the k-th's top digit and the count above it, for the gather and the finish
// of launches with many rows (each of their waves would otherwise read the row histogram).
__global__ __launch_bounds__(64) void select_digit_kernel(SelectArgs a) {
    const int r = blockIdx.x;
    int64_t t, C;
    row_info(a, r, &t, &C);
    if (C <= a.k_global) return;
    uint32_t b1, above1;
    wave_find_digit<kHistBins>(a.rowhist + (int64_t)r * kHistBins, (uint32_t)a.k_global, b1, above1);
    if (threadIdx.x == 0) {
        a.digits[2 * (int64_t)r] = b1;
        a.digits[2 * (int64_t)r + 1] = above1;
    }
}

// seven waves per SIMD for launches of many rows (query chunks run tens of thousands of these
// workgroups, which take their digit from select_digit_kernel); launches of a few long rows (decode)
// search the digit in every wave and hold the row histogram in registers meanwhile
template <bool GIVEN>
__global__ __launch_bounds__(256, GIVEN ? 7 : 4) void select_gather_kernel(SelectArgs a) {
    __shared__ GatherLds S;
    select_gather_body<GIVEN>(a, blockIdx.x, blockIdx.y, S);
}

// eight waves per SIMD: two workgroups per CU (LDS allows two) for the many rows of query chunks
template <bool GIVEN>
__global__ __launch_bounds__(kFinThreads, 8) void select_finish_kernel(SelectArgs a) {
    __shared__ FinishLds<kFinThreads> S;
    select_finish_body<kFinThreads, GIVEN>(a, blockIdx.x, S);
}

hipError_t launch_select(const SelectArgs& a, bool hist_done, hipStream_t s) {
    dim3 grid(a.R, a.nseg);
    if (!hist_done) {
        ProfScope ps("select_hist", s);
        select_hist_kernel<<<grid, 256, 0, s>>>(a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // launches of many rows find each row's digit once; a few long rows (decode) search it in
    // every workgroup instead of paying for one more launch
    const bool given = a.digits && a.R >= kSelDigitRows;
    if (given) {
        ProfScope ps("select_digit", s);
        select_digit_kernel<<<a.R, 64, 0, s>>>(a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    {
        ProfScope ps("select_gather", s);
        if (given) select_gather_kernel<true><<<grid, 256, 0, s>>>(a);
        else select_gather_kernel<false><<<grid, 256, 0, s>>>(a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // the finish reads the digit from a.digits, written by select_digit_kernel or by the gather
    ProfScope ps("select_finish", s);
    if (a.digits) select_finish_kernel<true><<<a.R, kFinThreads, 0, s>>>(a);
    else select_finish_kernel<false><<<a.R, kFinThreads, 0, s>>>(a);
    return hipGetLastError();
}

// ---- block-level selection -----------------------------------------------------------------
//
// The first-generation variant (kucoin news flash; lynxflow "Token-Level Sparse Selection"):
// candidates in consecutive blocks of `block` positions, a block kept whole when any member is
// important.  With the same score and budget: block score = the largest member score, the
// k_blocks best blocks by (block score desc, block id asc), expanded to their positions in the
// token index layout (a last block past the candidate count is cut there), then the window.

// Block maxima of one 4096-position segment of a row: thread x of the workgroup reads positions
// j0 + x + 256u, so a wave covers 64 consecutive positions per load and the `block` lanes of a
// block (block divides 64) fold their maximum in vector registers (group_max_nonneg).
constexpr int kBmSeg = 4096;

__global__ __launch_bounds__(256) void block_max_kernel(SelectArgs a) {
    const int r = blockIdx.x;
    int64_t t, C;
    row_info(a, r, &t, &C);
    const int64_t j0 = (int64_t)blockIdx.y * kBmSeg;
    if (j0 >= C) return;
    const float* sc = a.scores + (int64_t)r * a.cstride;
    float* bs = a.bscore + (int64_t)r * a.bstride;
    const int lane = threadIdx.x & 63;
    constexpr int PER = kBmSeg / 256;
    float v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int64_t j = j0 + u * 256 + threadIdx.x;
        v[u] = j < C ? sc[j] : -1.0f;            // scores are >= 0; -1 marks a position past C
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) v[u] = group_max_nonneg(v[u], a.block);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int64_t j = j0 + u * 256 + threadIdx.x;
        if ((lane & (a.block - 1)) == 0 && j < C) bs[j / a.block] = v[u];
    }
}

// One workgroup per row: exact radix select of the k_blocks-th best block maximum over the row's
// nb <= kBlkMaxCand blocks (held in registers, 16 per thread), then one ordered pass that keeps
// the blocks above it and the lowest-id ties, writes the block ids ascending and expands them.
constexpr int kBsThreads = 1024;
constexpr int kBsPer = kBlkMaxCand / kBsThreads;

__global__ __launch_bounds__(kBsThreads) void block_select_kernel(SelectArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t hist[kHistBins];
    __shared__ int32_t sel[4096];
    __shared__ uint32_t tmp[kBsThreads / 64 + 1];
    __shared__ uint32_t res[2];
    const int r = blockIdx.x;
    const int KB = a.k_blocks, blk = a.block, K = KB * blk, W = a.window;
    int64_t t, C;
    row_info(a, r, &t, &C);
    int32_t* irow = a.idx + (int64_t)r * (K + W);
    int32_t* brow = a.block_idx + (int64_t)r * KB;
    const int nb = (int)((C + blk - 1) / blk);

    for (int w = threadIdx.x; w < W; w += kBsThreads) {
        const int64_t first = t - W + 1 > 0 ? t - W + 1 : 0;
        const int64_t jj = first + w;
        irow[K + w] = (t >= 0 && jj <= t) ? (int32_t)jj : -1;
    }
    if (a.scores_dbg) {
        const float* sc = a.scores + (int64_t)r * a.cstride;
        float* dbg = a.scores_dbg + (int64_t)r * a.Nmax;
        for (int64_t j = threadIdx.x; j < a.Nmax; j += kBsThreads) dbg[j] = j < C ? sc[j] : -1.0f;
    }
    if (nb <= KB) {
        // every candidate block: positions 0 .. C-1 in order
        for (int x = threadIdx.x; x < KB; x += kBsThreads) brow[x] = x < nb ? x : -1;
        for (int x = threadIdx.x; x < K; x += kBsThreads) irow[x] = x < C ? x : -1;
        return;
    }
    const float* bs = a.bscore + (int64_t)r * a.bstride;
    uint32_t key[kBsPer];
#pragma unroll
    for (int u = 0; u < kBsPer; ++u) {
        const int b = u * kBsThreads + threadIdx.x;
        key[u] = b < nb ? __float_as_uint(bs[b]) : 0u;
    }
    // digit 1 [31:21]
    for (int x = threadIdx.x; x < kHistBins; x += kBsThreads) hist[x] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kBsPer; ++u)
        if (u * kBsThreads + (int)threadIdx.x < nb) atomicAdd(&hist[dig1(key[u])], 1u);
    __syncthreads();
    uint32_t b1, b2, b3, above1, above2, above3;
    block_find_digit<kBsThreads>(hist, kHistBins, (uint32_t)KB, b1, above1, tmp, res);
    const uint32_t k1 = (uint32_t)KB - above1;
    // digit 2 [20:10] among the keys of the k-th's digit-1 bucket
    for (int x = threadIdx.x; x < kHistBins; x += kBsThreads) hist[x] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kBsPer; ++u)
        if (u * kBsThreads + (int)threadIdx.x < nb && dig1(key[u]) == b1) atomicAdd(&hist[dig2(key[u])], 1u);
    __syncthreads();
    block_find_digit<kBsThreads>(hist, kHistBins, k1, b2, above2, tmp, res);
    const uint32_t k2 = k1 - above2;
    // digit 3 [9:0]
    for (int x = threadIdx.x; x < kHistBins; x += kBsThreads) hist[x] = 0;
    __syncthreads();
    const uint32_t pre = (b1 << 11) | b2;
#pragma unroll
    for (int u = 0; u < kBsPer; ++u)
        if (u * kBsThreads + (int)threadIdx.x < nb && (key[u] >> 10) == pre) atomicAdd(&hist[dig3(key[u])], 1u);
    __syncthreads();
    block_find_digit<kBsThreads>(hist, 1024, k2, b3, above3, tmp, res);
    const uint32_t need_eq = k2 - above3;            // ties at the threshold still needed
    const uint32_t T = (b1 << 21) | (b2 << 10) | b3;

    // ordered pass over block ids: rank ties and picks with running block scans
    uint32_t run_eq = 0, run_pick = 0;
#pragma unroll
    for (int u = 0; u < kBsPer; ++u) {
        if (u * kBsThreads >= nb) break;                 // uniform over the workgroup
        const int b = u * kBsThreads + threadIdx.x;
        const bool valid = b < nb;
        const bool eq = valid && key[u] == T;
        uint32_t tot_eq;
        const uint32_t er = run_eq + block_excl_scan<kBsThreads>(eq ? 1u : 0u, tmp, &tot_eq);
        const bool pick = valid && (key[u] > T || (eq && er < need_eq));
        uint32_t tot_pick;
        const uint32_t pos = run_pick + block_excl_scan<kBsThreads>(pick ? 1u : 0u, tmp, &tot_pick);
        if (pick && pos < (uint32_t)KB) sel[pos] = b;
        run_eq += tot_eq;
        run_pick += tot_pick;
    }
    __syncthreads();
    const int np = run_pick < (uint32_t)KB ? (int)run_pick : KB;   // == KB unless the counts disagreed
    for (int x = threadIdx.x; x < KB; x += kBsThreads) brow[x] = x < np ? sel[x] : -1;
    // expansion: only the highest block id (the last one picked) can be cut at C
    for (int x = threadIdx.x; x < K; x += kBsThreads) {
        const int i = x / blk;
        int32_t v = -1;
        if (i < np) {
            const int64_t j = (int64_t)sel[i] * blk + (x - i * blk);
            v = j < C ? (int32_t)j : -1;
        }
        irow[x] = v;
    }
}

// maxima_done: the score pass already wrote the block maxima (64-key blocks of query chunks)
hipError_t launch_select_blocks(const SelectArgs& a, bool maxima_done, hipStream_t s) {
    if (!maxima_done) {
        ProfScope ps("select_block_max", s);
        dim3 grid(a.R, (unsigned)((a.Nmax + kBmSeg - 1) / kBmSeg));
        block_max_kernel<<<grid, 256, 0, s>>>(a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    ProfScope ps("select_blocks", s);
    block_select_kernel<<<a.R, kBsThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace hs2
