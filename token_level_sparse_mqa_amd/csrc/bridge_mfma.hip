// KV-Bridge projection on MFMA: [K | V] = hidden . [Wk | Wv], one bf16 rounding at the end.
//
// KV Bridging (lynxflow blog, "Two-Level KV Sharing"; ainews page, mechanism paragraph): the
// cross-decoder full-attention layer's K/V cache is projected from self-decoder hidden states
// by the layer's own projections.  At the prefill-exit shape (T = 262144 tokens, D = 2048,
// d = 128) the product streams 1.07 GB of hidden states against 1 MB of weights, so it is
// bound by HBM: one pass over the hidden states, the weights served from L2.
//
// A workgroup owns 256 token rows and all 2d output columns (K and V together, so the hidden
// states are read once): eight waves in a 2 x 4 grid at d = 128, each with 128 rows x 64 columns
// of fp32 accumulators (4 x 2 MFMA blocks: per 16 reduction steps a wave reads 4 hidden operands
// at the full LDS rate and 2 weight operands through the half-rate transposed reads, 20% fewer
// LDS cycles than 2 x 4 blocks), 2 x 4 waves of 128 x 32 at d = 64.  The reduction over D runs
// in chunks of 64.  Hidden-state chunks [256 x 64] (three LDS buffers) and weight chunks [64 x 2d]
// (two at d = 128, three at d = 64) go from memory straight into LDS, so no registers hold loads
// in flight and two hidden chunks stream in while one is multiplied.  A operands are hidden-state
// rows (8 consecutive d per lane); B operands come from the row-major weight chunk through
// ds_read_b64_tr_b16.
#include "mfma_tiles.h"

namespace hs2 {

constexpr int kBrM = 256;          // token rows per workgroup
constexpr int kBrThreads = 512;    // eight waves
constexpr int kBrK = 64;           // reduction chunk

template <int DD, int BK>   // output columns per projection, reduction chunk
struct BrGeom {
    static constexpr int N = 2 * DD;                 // K and V columns
    static constexpr int HROW = BK * 2;              // bytes per hidden-state row in LDS
    static constexpr int HCPR = BK / 8;              // 16-byte chunks per hidden row
    static constexpr int HRPB = 256 / HROW;          // hidden rows per 256-byte bank cycle
    static constexpr int WROW = N * 2;               // bytes per weight row in LDS
    static constexpr int WCPR = N / 8;               // 16-byte chunks per weight row
    static constexpr int HBYTES = kBrM * HROW;
    static constexpr int WBYTES = BK * WROW;
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

// The reduction chunk that workgroup blockIdx.x takes at step kc.  If every workgroup walked the
// chunks in the same order, the 256 resident workgroups would all read the same 64- or 128-byte
// column slice of their 4 KB hidden rows (and the same weight rows) at once, which concentrates the
// requests on a few memory channels; starting each workgroup's walk 5 chunks after the previous
// workgroup's spreads them (measured on the prefill-exit shape: the loads alone 337 -> 269 us).
// The sum over the chunks is then taken in a rotated order, a different fp32 rounding order per
// workgroup; integer-valued operands stay exact.
__device__ __forceinline__ int stagger_chunk(int kc, int nk) {
    return (int)(((uint32_t)kc + blockIdx.x * 5u) % (uint32_t)nk);
}

// Loads into LDS: global_load_lds_dwordx4 writes lane i's 16 bytes at bytes [16 i, 16 i + 16) of a
// 1 KB block whose base is wave-uniform.  A block's lanes fetch the global chunks that belong at
// their LDS slots under the XOR swizzles above, so the operand reads see the swizzled layout.
typedef __attribute__((address_space(3))) char lds_char_t;

// One wave-wide load of 16 bytes per lane into LDS bytes [lds, lds + 1024) (lds wave-uniform),
// lane i's bytes at lds + 16 i: from `base + off` (uniform base, per-lane 32-bit offset), or from a
// per-lane address.  Written as inline asm so that the compiler does not take every later LDS read
// for a possible reader of these bytes and wait for all loads before it: the kernel orders them
// itself (s_waitcnt vmcnt, then a workgroup barrier, before a stage is read).  The instruction has
// no register results; its address registers are read when it issues.  M0 (the LDS base) is saved
// and restored around it, since the compiler does not track M0 through inline asm.
__device__ __forceinline__ void dma16(const char* base, uint32_t off, uint32_t lds) {
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(off), "s"(base), "s"(lds) : "memory");
}
__device__ __forceinline__ void dma16(const char* addr, uint32_t lds) {
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(addr), "s"(lds) : "memory");
}

// s_waitcnt with only vmcnt = N (gfx9 encoding; expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Hidden-state chunks take NSH LDS buffers and weight chunks NSW (NSH or NSH - 1: the weights come
// from L2 with a shorter latency); the loads of chunk kc + NSH - 1 (hidden) and kc + NSW - 1
// (weights) are issued while chunk kc is multiplied, weights first.
template <int DD, int BK, int NSH, int NSW, int MB>
__global__ __launch_bounds__(kBrThreads, 1) void bridge_mfma_kernel(BridgeArgs a) {
    using G = BrGeom<DD, BK>;
    // waves in a WR x WC grid, each with MB x NB MFMA blocks of 32 x 32 (held transposed)
    constexpr int WR = kBrM / (32 * MB), WC = 8 / WR, NB = (2 * DD / 32) / WC;
    static_assert(WR * WC == 8 && NB * WC * 32 == 2 * DD, "wave grid");
    static_assert(NSW == NSH || NSW == NSH - 1, "weight buffers: NSH or NSH - 1");
    static_assert(NSW >= 2, "at least double buffering");
    constexpr int HBLK = G::HBYTES / 8192;                // 1 KB hidden blocks per wave and chunk
    constexpr int WBLK = G::WBYTES / 8192;                // 1 KB weight blocks per wave and chunk
    static_assert(G::HBYTES % 8192 == 0 && G::WBYTES % 8192 == 0, "chunk blocks per wave");
    // loads (per lane) issued after the later of a chunk's hidden and weight loads, once the loads of
    // the chunk NSH - 2 steps ahead are out: what may stay in flight when that chunk is needed
    constexpr int AFTER = NSW == NSH ? (NSH - 2) * (HBLK + WBLK) : HBLK + (NSH - 3) * (HBLK + WBLK);
    __shared__ __attribute__((aligned(1024))) char smem[NSH * G::HBYTES + NSW * G::WBYTES];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n = lane & 31, hb = lane >> 5;
    const int wm = w / WC, wn = w % WC;
    const int64_t m0 = (int64_t)blockIdx.x * kBrM;
    const int nk = a.D / BK;

    // per-lane source of each block this wave fills: the logical chunk that the swizzle places at
    // the lane's LDS slot (32-bit byte offsets from the workgroup's first hidden row; weight addresses)
    const char* hbase = (const char*)(a.hidden + m0 * a.D);
    uint32_t hsrc[HBLK];
#pragma unroll
    for (int x = 0; x < HBLK; ++x) {
        const int o = (w + 8 * x) * 1024 + 16 * lane;
        const int row = o / G::HROW, p = (o % G::HROW) >> 4;
        const int c = p ^ ((row / G::HRPB) & (G::HCPR - 1));
        const int64_t gr = m0 + row < a.T ? row : a.T - 1 - m0;
        hsrc[x] = (uint32_t)(gr * a.D * 2 + 16 * c);
    }
    const char* wsrc[WBLK];
#pragma unroll
    for (int x = 0; x < WBLK; ++x) {
        const int o = (w + 8 * x) * 1024 + 16 * lane;
        const int kr = o / G::WROW, p = (o % G::WROW) >> 4;
        const int c = p ^ (((kr & 3) << 2) | (((kr >> 2) & 1) << 1));
        const bool isk = c < G::WCPR / 2;
        const int cc = isk ? c : c - G::WCPR / 2;
        wsrc[x] = (const char*)(isk ? a.wk : a.wv) + (kr * DD * 2 + 16 * cc);
    }
    // chunk kc (clamped: loads issued past the end re-read the last chunk into a buffer that nothing
    // reads any more), taken in the workgroup's rotated order
    const uint32_t lds_h = (uint32_t)(size_t)(lds_char_t*)smem + __builtin_amdgcn_readfirstlane(w) * 1024;
    const uint32_t lds_w = lds_h + NSH * G::HBYTES;
    auto issue_h = [&](int kc) {
        const uint32_t sb = lds_h + (kc % NSH) * G::HBYTES;
        kc = stagger_chunk(kc < nk ? kc : nk - 1, nk);
#pragma unroll
        for (int x = 0; x < HBLK; ++x) dma16(hbase, hsrc[x] + (uint32_t)kc * BK * 2, sb + 8192 * x);
    };
    auto issue_w = [&](int kc) {
        const uint32_t sb = lds_w + (kc % NSW) * G::WBYTES;
        kc = stagger_chunk(kc < nk ? kc : nk - 1, nk);
#pragma unroll
        for (int x = 0; x < WBLK; ++x) dma16(wsrc[x] + (uint32_t)kc * BK * DD * 2, sb + 8192 * x);
    };

    f32x16_t acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x16_t{};

    // the steady-state issue order (weights of chunk j + NSW - 1, then hidden of chunk j + NSH - 1)
    // run for j = 1 - NSH .. -1, skipping chunks below 0
#pragma unroll
    for (int j = 1 - NSH; j < 0; ++j) {
        if (j + NSW - 1 >= 0) issue_w(j + NSW - 1);
        issue_h(j + NSH - 1);
    }
    const int g = lane >> 4, q = lane & 15;
    for (int kc = 0; kc < nk; ++kc) {
        // this wave's loads of chunk kc have landed once at most AFTER loads are outstanding; the
        // barrier then covers every wave's, and every wave is done with chunk kc - 1's buffers
        wait_vmcnt<AFTER>();
        __syncthreads();
        issue_w(kc + NSW - 1);
        issue_h(kc + NSH - 1);
        const char* hb_ = smem + (kc % NSH) * G::HBYTES;
        const char* wb_ = smem + NSH * G::HBYTES + (kc % NSW) * G::WBYTES;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8_t aop[MB];
#pragma unroll
            for (int i = 0; i < MB; ++i)
                aop[i] = *(const bf16x8_t*)(hb_ + G::hoff(32 * MB * wm + 32 * i + n, 2 * ks + hb));
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int col = 32 * NB * wn + 32 * j + 16 * (g & 1) + 4 * (q & 3);
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
                for (int i = 0; i < MB; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bop, aop[i], acc[i][j], 0, 0, 0);
            }
        }
    }
    wait_vmcnt<0>();      // the clamped loads past the end land before the workgroup ends

    // epilogue: bf16 (round to nearest even), staged through LDS so that global rows are written
    // whole.  The MFMAs take the weights as their first operand, so block (i, j) holds the
    // transposed product: lane (n, hb) has token 32 i + n and, for each q, the 4 consecutive output
    // columns 8 q + 4 hb + 0..3 (e = 4 q .. 4 q + 3), one 8-byte LDS write into the tile
    // [256 tokens][2d columns: K, then V] (rows padded by 8 bytes, so the 32 tokens of a write land
    // in 32 different bank pairs).  Then every thread copies 16-byte row chunks to K and V.
    constexpr int OST = 2 * DD * 2 + 8;                   // bytes per token row of the output tile
    static_assert(kBrM * OST <= NSH * G::HBYTES + NSW * G::WBYTES, "output tile fits the stage buffers");
    __syncthreads();                                      // every wave is done with the stages
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            char* trow = smem + (32 * MB * wm + 32 * i + n) * OST + (32 * NB * wn + 32 * j + 4 * hb) * 2;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc[i][j][4 * q]) |
                                    ((uint32_t)f32_to_bf16_rne(acc[i][j][4 * q + 1]) << 16);
                const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc[i][j][4 * q + 2]) |
                                    ((uint32_t)f32_to_bf16_rne(acc[i][j][4 * q + 3]) << 16);
                *(u32x2_t*)(trow + 16 * q) = u32x2_t{lo, hi};
            }
        }
    __syncthreads();
    // 16-byte chunks: 2d / 8 per token row (K's d / 8 first); rows past T are skipped
    constexpr int CPR = 2 * DD / 8;
    const bool st16 = (a.stride & 7) == 0 && ((uintptr_t)a.k_out & 15) == 0 && ((uintptr_t)a.v_out & 15) == 0;
    for (int x = tid; x < kBrM * CPR; x += kBrThreads) {
        const int r = x / CPR, c = x % CPR;
        const int64_t row = m0 + r;
        if (row >= a.T) continue;
        const u32x4_t v = *(const u32x4_t*)(smem + r * OST + 16 * c);
        uint16_t* dst = (c < CPR / 2 ? a.k_out + 8 * c : a.v_out + 8 * (c - CPR / 2)) + row * a.stride;
        if (st16) {
            *(u32x4_t*)dst = v;
        } else {
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) { dst[2 * w2] = (uint16_t)v[w2]; dst[2 * w2 + 1] = (uint16_t)(v[w2] >> 16); }
        }
    }
}

hipError_t launch_bridge_mfma(const BridgeArgs& a, hipStream_t s) {
    ProfScope ps("bridge_mfma", s);
    dim3 grid((unsigned)((a.T + kBrM - 1) / kBrM));
    // 160 KB of LDS at d = 128 (3 hidden + 2 weight buffers of 32 KB), 144 KB at d = 64 (3 + 3)
    if (a.d == 128) bridge_mfma_kernel<128, kBrK, 3, 2, 4><<<grid, kBrThreads, 0, s>>>(a);
    else bridge_mfma_kernel<64, kBrK, 3, 3, 4><<<grid, kBrThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace hs2
