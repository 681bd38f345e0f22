// The whole decode hybrid block in one launch: the full-attention layer over the key splits, the
// merge of the splits (o and the per-head log-sum-exp), the selection scores, the top-k
// selection with the window, and every sparse layer of the block over the selected rows with its
// own merge (lynxflow blog, "Two-Level KV Sharing": the sparse layers reuse the full layer's cache
// and indices; ainews page, closing paragraph: the compute saving on paper becomes a wall-clock
// saving only through the kernels, the memory traffic and the launch order).
//
// A cooperative launch of exactly as many workgroups as fit on the GPU at once (the runtime
// refuses a launch that cannot be resident).  Each phase is a list of work items (the workgroups
// of the separate kernels: the same device code, see the *_dev.h headers) taken round-robin by
// the resident workgroups; a grid-wide barrier separates the phases, since every item of a phase
// may read what any item of the previous one wrote.  All workgroups run the same phase loops, so
// every one of them reaches every barrier (the runtime's grid barrier of cooperative groups).  The
// selection finish runs with the common 256 threads instead of its kernel's 1024.
#include "attn_combine_dev.h"
#include "attn_rows_dev.h"
#include "score_rows_dev.h"
#include "select_dev.h"

#include <hip/hip_cooperative_groups.h>

namespace hs2 {

constexpr int kDbThreads = kRowWaves * 64;
template <int D>
union DecodeLds {
    RowLds<D> rows;
    CombineWideLds cw;
    ScoreLds sc;
    GatherLds ga;
    FinishLds<kDbThreads> fin;
};

// Merge of the key splits of `a` (block rows nrow): the narrow or wide form, as the separate
// combine launch would choose it.
template <int D>
__device__ __forceinline__ void db_combine(const AttnArgs& a, int nrow, DecodeLds<D>& S) {
    const int H = a.H;
    if (a.nsplit > kCombineNarrowMax) {
        constexpr int NZ = D / 16;
        const int n = nrow * H * NZ;
        for (int it = blockIdx.x; it < n; it += gridDim.x) {
            combine_wide_body<D>(a, it / (H * NZ), (it / NZ) % H, it % NZ, S.cw);
            __syncthreads();
        }
    } else {
        const int n = nrow * H;
        for (int it = blockIdx.x; it < n; it += gridDim.x)
            if ((int)threadIdx.x < D) combine_narrow_body<D>(a, it / H, it % H);
    }
}

template <int D, int KV>
__global__ __launch_bounds__(kDbThreads, 2) void decode_block_kernel(DecodeBlockArgs p) {
    __shared__ __attribute__((aligned(16))) DecodeLds<D> S;
    cooperative_groups::grid_group grid = cooperative_groups::this_grid();
    const int R = p.full.B * p.full.Tq;
    const int G = gridDim.x;

    // full layer: (row, key split) items; split 0 of a row clears its selection workspace
    for (int it = blockIdx.x; it < R * p.full.nsplit; it += G) {
        attn_rows_body<D, KV, false>(p.full, it / p.full.nsplit, it % p.full.nsplit, S.rows);
        __syncthreads();
    }
    grid.sync();
    if (p.full.nsplit > 1) {
        db_combine<D>(p.full, R, S);
        grid.sync();
    }
    // selection scores: (row, split) items, with the row histograms of the top radix digit
    for (int it = blockIdx.x; it < R * p.score.nsplit; it += G) {
        score_rows_body<D, KV>(p.score, it / p.score.nsplit, it % p.score.nsplit, S.sc);
        __syncthreads();
    }
    grid.sync();
    // top-k: (row, segment) gather items, then one finish item per row
    for (int it = blockIdx.x; it < R * p.sel.nseg; it += G) {
        select_gather_body(p.sel, it / p.sel.nseg, it % p.sel.nseg, S.ga);
        __syncthreads();
    }
    grid.sync();
    for (int it = blockIdx.x; it < R; it += G) {
        select_finish_body<kDbThreads>(p.sel, it, S.fin);
        __syncthreads();
    }
    grid.sync();
    // sparse layers: (layer * R + row, split) items over the selected rows, then their merge
    const int RL = R * p.sparse.nlayer;
    for (int it = blockIdx.x; it < RL * p.sparse.nsplit; it += G) {
        attn_rows_body<D, KV, true>(p.sparse, it / p.sparse.nsplit, it % p.sparse.nsplit, S.rows);
        __syncthreads();
    }
    if (p.sparse.nsplit > 1) {
        grid.sync();
        db_combine<D>(p.sparse, RL, S);
    }
}

template <int D, int KV>
hipError_t launch_db(const DecodeBlockArgs& a, hipStream_t s) {
    static int grid_size = 0;          // resident workgroups: occupancy x compute units (first call)
    if (grid_size == 0) {
        int dev = 0, ncu = 0, per = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, decode_block_kernel<D, KV>, kDbThreads, 0);
        if (e != hipSuccess) return e;
        if (per < 1 || ncu < 1) return hipErrorCooperativeLaunchTooLarge;
        grid_size = per * ncu;
    }
    DecodeBlockArgs args = a;
    void* kargs[] = {&args};
    return hipLaunchCooperativeKernel((const void*)decode_block_kernel<D, KV>, dim3(grid_size), dim3(kDbThreads),
                                      kargs, 0, s);
}

hipError_t launch_decode_block(const DecodeBlockArgs& a, hipStream_t s) {
    ProfScope ps("decode_block", s);
    if (a.full.kv_dtype == HS2_FP8_E4M3)
        return a.full.d == 128 ? launch_db<128, HS2_FP8_E4M3>(a, s) : launch_db<64, HS2_FP8_E4M3>(a, s);
    return a.full.d == 128 ? launch_db<128, HS2_BF16>(a, s) : launch_db<64, HS2_BF16>(a, s);
}

}  // namespace hs2
