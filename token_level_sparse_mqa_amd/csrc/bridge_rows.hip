// KV-Bridge projection for a few token rows: [K | V] = hidden . [Wk | Wv], one bf16 rounding.
//
// KV Bridging (lynxflow blog, "Two-Level KV Sharing"; ainews page, mechanism paragraph): the
// cross-decoder full layer's K/V rows come from self-decoder hidden states through the layer's
// own projections.  In the agentic loop a decoded action token appends one row at a time
// (agentik-os article, section 1 "Agentic inference as the driving workload"), so the product is a
// vector-matrix product that must read the 2 * D * d bf16 weights once; the MFMA tile kernel
// (256 rows per workgroup, all 2d columns in one workgroup) would run one workgroup for it.
//
// Here a workgroup owns 32 output columns of one projection (64 contiguous bytes of every weight
// row) and RT token rows; the grid is (2d / 32 column blocks) x ceil(T / RT).  Four lanes cover
// one weight row's 64 bytes, 64 row groups stride through D, so every weight byte of the block is
// read once, in 16-byte loads.  The token rows are staged transposed in LDS (the RT values of one
// reduction index in one read).  Partial sums over the 64 row groups are folded with halving
// exchanges inside each wave (every step sends half of what a lane holds) and summed over the
// four waves through LDS.  fp32 accumulation in any order, then bf16 round to nearest even.
#include "hs2_device.h"
#include "mfma_tiles.h"

namespace hs2 {

constexpr int kBrRowsThreads = 256;
constexpr int kBrRowsCols = 32;       // output columns per workgroup
constexpr int kBrRowsMaxD = 4096;     // hidden width staged in LDS
constexpr int kBrRowsMaxT = 64;       // spans up to this many rows take this kernel

// One halving step of the in-wave fold: v[0, 2H) -> v[0, H); lanes with `mask` set keep the upper half.
template <int H>
__device__ __forceinline__ void fold_half(float* v, int mask, int lane) {
    const bool up = (lane & mask) != 0;
#pragma unroll
    for (int j = 0; j < H; ++j) {
        const float send = up ? v[j] : v[j + H];
        const float keep = up ? v[j + H] : v[j];
        v[j] = keep + __shfl_xor(send, mask);
    }
}

template <int DD, int RT>
__global__ __launch_bounds__(kBrRowsThreads) void bridge_rows_kernel(BridgeArgs a) {
    constexpr int N = RT * 8;                       // partial sums per lane: RT rows x 8 columns
    // values per lane after the folds over lane bits 5, 4, 3, 2 (while more than one is left)
    constexpr int E = N >= 16 ? N / 16 : 1;
    __shared__ __align__(16) uint16_t ht[kBrRowsMaxD * RT];   // ht[i * RT + t] = hidden[row0 + t][i]
    __shared__ float red[4][64][E];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    constexpr int CB = DD / kBrRowsCols;            // column blocks per projection
    const int mat = blockIdx.x / CB, col0 = (blockIdx.x % CB) * kBrRowsCols;
    const int64_t row0 = (int64_t)blockIdx.y * RT;
    const int D = a.D;

    // stage the RT hidden rows transposed (rows past T are zero)
    for (int c = tid; c < D / 8; c += kBrRowsThreads) {
        u32x4_t h[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t)
            h[t] = row0 + t < a.T ? *(const u32x4_t*)(a.hidden + (row0 + t) * D + 8 * c) : u32x4_t{0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            uint16_t* dst = ht + (8 * c + k) * RT;
#pragma unroll
            for (int t = 0; t < RT; ++t) dst[t] = (uint16_t)(h[t][k >> 1] >> (16 * (k & 1)));
        }
    }
    __syncthreads();

    const int q = tid & 3, rg = tid >> 2;           // 8-column quarter, row group
    const uint16_t* wm = (mat == 0 ? a.wk : a.wv) + col0 + 8 * q;
    float acc[N];
#pragma unroll
    for (int j = 0; j < N; ++j) acc[j] = 0.f;
    const int nrow = D / 64;
#pragma unroll 8
    for (int s = 0; s < nrow; ++s) {
        const int i = rg + 64 * s;
        const u32x4_t wr = *(const u32x4_t*)(wm + (int64_t)i * DD);
        float wf[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) wf[k] = bf16_to_f32((uint16_t)(wr[k >> 1] >> (16 * (k & 1))));
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            const float hv = bf16_to_f32(ht[i * RT + t]);
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[8 * t + k] = fmaf(hv, wf[k], acc[8 * t + k]);
        }
    }

    // fold over the wave's 16 row groups (lane bits 5..2); a lane keeps E values
    if constexpr (N >= 2) fold_half<N / 2>(acc, 32, lane);
    if constexpr (N >= 4) fold_half<N / 4>(acc, 16, lane); else acc[0] += __shfl_xor(acc[0], 16);
    if constexpr (N >= 8) fold_half<N / 8>(acc, 8, lane); else acc[0] += __shfl_xor(acc[0], 8);
    if constexpr (N >= 16) fold_half<N / 16>(acc, 4, lane); else acc[0] += __shfl_xor(acc[0], 4);
#pragma unroll
    for (int e = 0; e < E; ++e) red[w][lane][e] = acc[e];
    __syncthreads();

    // lane L holds the sums j = off(L) + e of its quarter, off(L) = sum over the halving steps of
    // (bit set ? half : 0); lanes that only differ in a plain-add bit hold the same values
    for (int x = tid; x < 64 * E; x += kBrRowsThreads) {
        const int L = x / E, e = x % E;
        int off = 0;
        if (N >= 2) off += (L & 32) ? N / 2 : 0;
        if (N >= 4) off += (L & 16) ? N / 4 : 0; else if (L & 16) continue;
        if (N >= 8) off += (L & 8) ? N / 8 : 0; else if (L & 8) continue;
        if (N >= 16) off += (L & 4) ? N / 16 : 0; else if (L & 4) continue;
        const int j = off + e, t = j >> 3;
        const int64_t row = row0 + t;
        if (row >= a.T) continue;
        const float sum = red[0][L][e] + red[1][L][e] + red[2][L][e] + red[3][L][e];
        uint16_t* out = mat == 0 ? a.k_out : a.v_out;
        out[row * a.stride + col0 + 8 * (L & 3) + (j & 7)] = f32_to_bf16_rne(sum);
    }
}

bool bridge_rows_fits(const BridgeArgs& a) { return a.T <= kBrRowsMaxT && a.D <= kBrRowsMaxD; }

hipError_t launch_bridge_rows(const BridgeArgs& a, hipStream_t s) {
    ProfScope ps("bridge_rows", s);
    const int RT = a.T == 1 ? 1 : 4;
    dim3 grid((unsigned)(2 * a.d / kBrRowsCols), (unsigned)((a.T + RT - 1) / RT));
    if (a.d == 128) {
        if (RT == 1) bridge_rows_kernel<128, 1><<<grid, kBrRowsThreads, 0, s>>>(a);
        else bridge_rows_kernel<128, 4><<<grid, kBrRowsThreads, 0, s>>>(a);
    } else {
        if (RT == 1) bridge_rows_kernel<64, 1><<<grid, kBrRowsThreads, 0, s>>>(a);
        else bridge_rows_kernel<64, 4><<<grid, kBrRowsThreads, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace hs2
