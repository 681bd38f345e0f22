// KV-Bridge projection on MFMA: [K | V] = hidden . [Wk | Wv], one bf16 rounding at the end.
//
// KV Bridging (lynxflow blog, "Two-Level KV Sharing"; ainews page, mechanism paragraph): the
// cross-decoder full-attention layer's K/V cache is projected from self-decoder hidden states
// by the layer's own projections.  At the prefill-exit shape (T = 262144 tokens, D = 2048,
// d = 128) the product streams 1.07 GB of hidden states against 1 MB of weights, so it is
// bound by HBM: one pass over the hidden states, the weights served from L2.
//
// A workgroup owns 256 token rows and all 2d output columns (K and V together, so the hidden
// states are read once): eight waves in a 4 x 2 grid, each with 64 rows x d columns of fp32
// accumulators (2 x 4 MFMA blocks at d = 128, which keeps the LDS operand reads per MFMA low).
// The reduction over D runs in chunks of 64: the hidden-state chunk [256 x 64] and the weight
// chunk [64 x 2d] are staged in LDS (double-buffered), with the global loads of the next
// chunks in flight in registers.  A operands are hidden-state rows (8 consecutive d per lane);
// B operands come from the row-major weight chunk through ds_read_b64_tr_b16.
#include "mfma_tiles.h"

namespace hs2 {

constexpr int kBrM = 256;          // token rows per workgroup
constexpr int kBrThreads = 512;    // eight waves
constexpr int kBrK = 64;           // reduction chunk
constexpr int kBrStages = 2;       // chunks in flight in registers (deeper pipelines measured slower)

template <int DD, int BK>   // output columns per projection, reduction chunk
struct BrGeom {
    static constexpr int N = 2 * DD;                 // K and V columns
    static constexpr int MB = 2;                     // MFMA row blocks per wave (64 rows)
    static constexpr int NB = DD / 32;               // MFMA column blocks per wave (d columns)
    static constexpr int HROW = BK * 2;              // bytes per hidden-state row in LDS
    static constexpr int HCPR = BK / 8;              // 16-byte chunks per hidden row
    static constexpr int HRPB = 256 / HROW;          // hidden rows per 256-byte bank cycle
    static constexpr int WROW = N * 2;               // bytes per weight row in LDS
    static constexpr int WCPR = N / 8;               // 16-byte chunks per weight row
    static constexpr int HBYTES = kBrM * HROW;
    static constexpr int WBYTES = BK * WROW;
    static constexpr int HCH = kBrM * HCPR;          // 16-byte chunks of a hidden chunk
    static constexpr int WCH = BK * WCPR;            // 16-byte chunks of a weight chunk
    static constexpr int HX = HCH / kBrThreads;
    static constexpr int WX = (WCH + kBrThreads - 1) / kBrThreads;
    // An operand read covers 16 hidden rows (16 lanes, one chunk each), HRPB rows to a bank cycle:
    // chunk XOR ((row / HRPB) mod HCPR) gives them 16 different bank groups.
    __device__ static __forceinline__ int hoff(int row, int chunk) {
        return row * HROW + ((chunk ^ ((row / HRPB) & (HCPR - 1))) << 4);
    }
    // Weight rows are read transposed: the two 16-lane groups of a half wave read the same 4 rows,
    // the second group's chunk pair 2 chunks after the first's.  XOR 4 (row mod 4) + 2 ((row / 4)
    // mod 2) keeps bit 1 equal over the 4 rows, so the 8 pairs land in 8 different bank groups.
    __device__ static __forceinline__ int woff(int row, int chunk) {
        return row * WROW + ((chunk ^ (((row & 3) << 2) | (((row >> 2) & 1) << 1))) << 4);
    }
};

// BK-deep reduction chunks, NST of them in flight in registers: a chunk's loads are issued
// NST - 1 chunks before it is stored to LDS, so NST - 1 chunk computations hide their latency.
template <int DD, int BK, int NST>
__global__ __launch_bounds__(kBrThreads, 1) void bridge_mfma_kernel(BridgeArgs a) {
    using G = BrGeom<DD, BK>;
    __shared__ __attribute__((aligned(16))) char hs[2][G::HBYTES];
    __shared__ __attribute__((aligned(16))) char ws[2][G::WBYTES];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n = lane & 31, hb = lane >> 5;
    const int wm = w >> 1, wn = w & 1;                 // wave rows [64 wm, +64), columns [d wn, +d)
    const int64_t m0 = (int64_t)blockIdx.x * kBrM;
    const int nk = a.D / BK;

    // per-thread load slots: 32-bit byte offsets from the workgroup's first hidden row / weights
    const char* hbase = (const char*)(a.hidden + m0 * a.D);
    uint32_t hoffs[G::HX];
    int hst[G::HX];
#pragma unroll
    for (int x = 0; x < G::HX; ++x) {
        const int q = tid + x * kBrThreads;
        const int row = q / G::HCPR, c = q % G::HCPR;
        const int64_t gr = m0 + row < a.T ? row : a.T - 1 - m0;
        hoffs[x] = (uint32_t)(gr * a.D * 2 + 16 * c);
        hst[x] = G::hoff(row, c);
    }
    uint32_t woffs[G::WX];
    int wst[G::WX];
    bool wisk[G::WX];
#pragma unroll
    for (int x = 0; x < G::WX; ++x) {
        int q = tid + x * kBrThreads;
        q = q < G::WCH ? q : G::WCH - 1;
        const int kr = q / G::WCPR, c = q % G::WCPR;      // c < WCPR/2: Wk, else Wv
        wisk[x] = c < G::WCPR / 2;
        const int cc = wisk[x] ? c : c - G::WCPR / 2;
        woffs[x] = (uint32_t)(kr * DD * 2 + 16 * cc);
        wst[x] = G::woff(kr, c);
    }
    u32x4_t rh[NST][G::HX], rw[NST][G::WX];
    auto load = [&](int st, int kc) {
        kc = kc < nk ? kc : nk - 1;
        const uint32_t hk = (uint32_t)kc * BK * 2;                 // bytes along a hidden row
        const uint32_t wk = (uint32_t)kc * BK * DD * 2;            // bytes down the weights
#pragma unroll
        for (int x = 0; x < G::HX; ++x) rh[st][x] = ld16<false>(hbase + (hoffs[x] + hk));
#pragma unroll
        for (int x = 0; x < G::WX; ++x)
            rw[st][x] = *(const u32x4_t*)((const char*)(wisk[x] ? a.wk : a.wv) + (woffs[x] + wk));
    };
    auto store = [&](int st, int buf) {
#pragma unroll
        for (int x = 0; x < G::HX; ++x) *(u32x4_t*)(hs[buf] + hst[x]) = rh[st][x];
#pragma unroll
        for (int x = 0; x < G::WX; ++x)
            if (tid + x * kBrThreads < G::WCH) *(u32x4_t*)(ws[buf] + wst[x]) = rw[st][x];
    };

    f32x16_t acc[G::MB][G::NB];
#pragma unroll
    for (int i = 0; i < G::MB; ++i)
#pragma unroll
        for (int j = 0; j < G::NB; ++j) acc[i][j] = f32x16_t{};

#pragma unroll
    for (int u = 0; u < NST; ++u) load(u, u);
    store(0, 0);
    __syncthreads();
    const int g = lane >> 4, q = lane & 15;
    // chunk kc from LDS buffer kc & 1, then register slot u + 1 into the other buffer and the loads
    // of chunk kc + NST into slot u
    auto step = [&](int kc, int u, bool store_next) {
        const int buf = kc & 1;
        const char* hb_ = hs[buf];
        const char* wb_ = ws[buf];
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            // A: hidden rows 64 wm + 32 i + n, d = 16 ks + 8 hb + {0..7}
            bf16x8_t aop[G::MB];
#pragma unroll
            for (int i = 0; i < G::MB; ++i)
                aop[i] = *(const bf16x8_t*)(hb_ + G::hoff(64 * wm + 32 * i + n, 2 * ks + hb));
#pragma unroll
            for (int j = 0; j < G::NB; ++j) {
                // B: weight rows d = 16 ks + 8 hb + 4 h + (q >> 2), columns wn*d + 32 j + 16 (g & 1) + 4 (q & 3)
                const int col = DD * wn + 32 * j + 16 * (g & 1) + 4 * (q & 3);
                u32x4_t r;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int krow = 16 * ks + 8 * (g >> 1) + 4 * h + (q >> 2);
                    const char* p = wb_ + G::woff(krow, col >> 3) + (col & 7) * 2;
                    const v4i16_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)p);
                    const u32x2_t tu = __builtin_bit_cast(u32x2_t, t);
                    r[2 * h] = tu[0];
                    r[2 * h + 1] = tu[1];
                }
                const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, r);
#pragma unroll
                for (int i = 0; i < G::MB; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[i], bop, acc[i][j], 0, 0, 0);
            }
        }
        if (store_next) store((u + 1) % NST, buf ^ 1);
        load(u, kc + NST);
        __syncthreads();
    };
    // Whole groups of NST chunks run without a branch: the store of the chunk after the last one
    // writes clamped loads into a buffer nothing reads any more.  A conditional store or an early
    // exit inside the group gives the loop several back edges with different loads in flight,
    // and the compiler's wait analysis then stalls each group on loads issued just before it.
    int kc = 0;
    for (; kc + NST <= nk; kc += NST) {
#pragma unroll
        for (int u = 0; u < NST; ++u) step(kc + u, u, true);
    }
#pragma unroll
    for (int u = 0; u < NST - 1; ++u)
        if (kc + u < nk) step(kc + u, u, kc + u + 1 < nk);

    // epilogue: bf16 (round to nearest even); wave column half 0 writes K, half 1 writes V
    uint16_t* out = wn == 0 ? a.k_out : a.v_out;
#pragma unroll
    for (int i = 0; i < G::MB; ++i)
#pragma unroll
        for (int j = 0; j < G::NB; ++j) {
            const int oc = 32 * j + n;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = m0 + 64 * wm + 32 * i + 8 * (e >> 2) + 4 * hb + (e & 3);
                if (row < a.T) out[row * a.stride + oc] = f32_to_bf16_rne(acc[i][j][e]);
            }
        }
}

hipError_t launch_bridge_mfma(const BridgeArgs& a, hipStream_t s) {
    ProfScope ps("bridge_mfma", s);
    dim3 grid((unsigned)((a.T + kBrM - 1) / kBrM));
    if (a.d == 128) bridge_mfma_kernel<128, kBrK, kBrStages><<<grid, kBrThreads, 0, s>>>(a);
    else bridge_mfma_kernel<64, kBrK, kBrStages><<<grid, kBrThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace hs2
