// Multi-target KV bridge into FP8 caches: for every target layer l,
//   x = hidden . W_l^T  (fp32 accumulation),  scale[t] = amax_c |x[t, c]| / 448,
//   code[t, c] = E4M3FN(x[t, c] / scale[t])   (round to nearest even, saturating at 448),
// for K and V alike.
//
// KV Bridging (lynxflow blog, "Two-Level KV Sharing"; ainews page, mechanism paragraph): each
// cross-decoder full-attention layer keeps its own K/V projections of the self-decoder's hidden
// states; the FP8 caches with a per-row scale follow the ainews page's experimental setup.  With
// every target reading the same hidden states, one launch serves all of them and the arithmetic
// intensity grows with the number of targets, past the HBM ridge: the kernel is built to be bound
// by the matrix cores.
//
// A workgroup computes 256 token rows x [K | V] (2d columns) of one target; the targets of a
// row tile run next to each other on one XCD, so the later ones find the tile's hidden states in
// that XCD's L2.  Weights come in a linear layer's layout (output rows [d, D]), so
// both MFMA operands are 8 consecutive reduction elements of one LDS row, read at full rate with
// ds_read_b128 (rows of 128 bytes, 16-byte chunks XOR-swizzled by row pair).  Eight waves in a
// 4 x 2 grid hold 64 rows x d columns each (K for wave column 0, V for 1), so a wave holds whole
// K or V rows and the per-row maximum is a fold over its own lanes.  The codes come from the
// packed fp32 -> E4M3FN conversion (nearest, ties to even), two per instruction.  The reduction runs in
// 64-deep chunks, double-buffered in LDS with the next chunk's loads in flight in registers.
#include "hs2_device.h"
#include "mfma_tiles.h"

#include <type_traits>

namespace hs2 {

constexpr int kB8M = 256;          // token rows per workgroup
constexpr int kB8Threads = 512;
constexpr int kB8K = 64;           // reduction chunk (128 bytes of a row)
constexpr int kB8Stages = 2;

// Byte offset of 16-byte chunk c (0..7) of LDS row r: two rows per 256-byte bank cycle, so the
// chunk index is XORed with the row pair number; 16 consecutive rows read at one chunk then hit
// 16 different bank groups.
__device__ __forceinline__ int b8_off(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

template <int DD>
__global__ __launch_bounds__(kB8Threads, 1) void bridge_fp8_kernel(BridgeFp8Args a) {
    constexpr int N = 2 * DD;                    // K and V columns of one target
    constexpr int NB = DD / 32;                  // MFMA column blocks per wave
    constexpr int HX = kB8M * 8 / kB8Threads;    // 16-byte hidden chunks per thread and chunk
    constexpr int WX = N * 8 / kB8Threads;       // 16-byte weight chunks per thread and chunk
    __shared__ __attribute__((aligned(16))) char hs[2][kB8M * 128];
    __shared__ __attribute__((aligned(16))) char ws[2][N * 128];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n = lane & 31, hb = lane >> 5;
    const int wm = w >> 1, wn = w & 1;
    // workgroup i runs on XCD i mod 8: XCD k takes the consecutive work items from k q + min(k, r)
    // (nwg = 8 q + r), so the targets of a row tile run on one XCD and share its L2
    const int nwg = gridDim.x, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int item = xcd * (nwg >> 3) + (xcd < (nwg & 7) ? xcd : (nwg & 7)) + slot;
    const int tgt = item % a.L;
    const int64_t m0 = (int64_t)(item / a.L) * kB8M;
    const int nk = a.D / kB8K;

    const char* hbase = (const char*)(a.hidden + m0 * a.D);
    uint32_t hoffs[HX];
    int hst[HX];
#pragma unroll
    for (int x = 0; x < HX; ++x) {
        const int q = tid + x * kB8Threads;
        const int row = q >> 3, c = q & 7;
        const int64_t gr = m0 + row < a.T ? row : a.T - 1 - m0;     // rows past T repeat the last
        hoffs[x] = (uint32_t)(gr * a.D * 2 + 16 * c);
        hst[x] = b8_off(row, c);
    }
    // the target's pointers, picked with static indices (a runtime index into the argument
    // arrays would copy them to scratch memory)
    const uint16_t *wkp = a.wk[0], *wvp = a.wv[0];
    uint8_t *kop = a.k_out[0], *vop = a.v_out[0];
    float *ksp = a.k_scale[0], *vsp = a.v_scale[0];
#pragma unroll
    for (int l = 1; l < kMaxTargets; ++l)
        if (tgt == l) {
            wkp = a.wk[l]; wvp = a.wv[l]; kop = a.k_out[l]; vop = a.v_out[l]; ksp = a.k_scale[l]; vsp = a.v_scale[l];
        }
    const char* wkb = (const char*)wkp;
    const char* wvb = (const char*)wvp;
    // slot x covers output columns 64 x .. 64 x + 63 (K then V), so whether it reads Wk or Wv is
    // known at compile time
    const uint32_t woff = (uint32_t)((tid >> 3) * a.D * 2 + 16 * (tid & 7));
    int wst[WX];
#pragma unroll
    for (int x = 0; x < WX; ++x) wst[x] = b8_off((tid >> 3) + 64 * x, tid & 7);
    u32x4_t rh[kB8Stages][HX], rw[kB8Stages][WX];
    auto load = [&](int st, int kc) {
        kc = kc < nk ? kc : nk - 1;
        const uint32_t kb = (uint32_t)kc * 128;
#pragma unroll
        for (int x = 0; x < HX; ++x) rh[st][x] = *(const u32x4_t*)(hbase + (hoffs[x] + kb));
#pragma unroll
        for (int x = 0; x < WX; ++x) {
            const char* wb = 64 * x < DD ? wkb + (size_t)(64 * x) * a.D * 2 : wvb + (size_t)(64 * x - DD) * a.D * 2;
            rw[st][x] = *(const u32x4_t*)(wb + (woff + kb));
        }
    };
    auto store = [&](int st, int buf) {
#pragma unroll
        for (int x = 0; x < HX; ++x) *(u32x4_t*)(hs[buf] + hst[x]) = rh[st][x];
#pragma unroll
        for (int x = 0; x < WX; ++x) *(u32x4_t*)(ws[buf] + wst[x]) = rw[st][x];
    };

    f32x16_t acc[2][NB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x16_t{};

#pragma unroll
    for (int u = 0; u < kB8Stages; ++u) load(u, u);
    store(0, 0);
    __syncthreads();
    // one chunk: MFMAs from LDS buffer kc & 1, then the next chunk's registers (stage ST ^ 1) go to
    // the other buffer and the chunk after it is loaded into stage ST
    auto chunk = [&](int kc, auto st_c) {
        constexpr int ST = decltype(st_c)::value;
        const int buf = kc & 1;
        const char* hp = hs[buf];
        const char* wp = ws[buf];
#pragma unroll
        for (int ks = 0; ks < kB8K / 16; ++ks) {
            // A: hidden row 64 wm + 32 i + n, reduction elements 16 ks + 8 hb .. +7
            bf16x8_t aop[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) aop[i] = *(const bf16x8_t*)(hp + b8_off(64 * wm + 32 * i + n, 2 * ks + hb));
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                // B: weight row (output column) d wn + 32 j + n, the same reduction elements
                const bf16x8_t bop = *(const bf16x8_t*)(wp + b8_off(DD * wn + 32 * j + n, 2 * ks + hb));
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[i], bop, acc[i][j], 0, 0, 0);
            }
        }
        if (kc + 1 < nk) store(ST ^ 1, buf ^ 1);
        load(ST, kc + kB8Stages);
        __syncthreads();
    };
    int kc = 0;
    for (; kc + 1 < nk; kc += 2) {
        chunk(kc, std::integral_constant<int, 0>{});
        chunk(kc + 1, std::integral_constant<int, 1>{});
    }
    if (kc < nk) chunk(kc, std::integral_constant<int, 0>{});

    // epilogue: the wave holds rows 64 wm + 32 i + 8 (e >> 2) + 4 hb + (e & 3), columns 32 j + n
    // of K (wn = 0) or V (wn = 1); the row maximum folds over j in the lane, then over the 32
    // lanes of the half wave
    uint8_t* out = wn == 0 ? kop : vop;
    float* sout = wn == 0 ? ksp : vsp;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            float m = 0.f;
#pragma unroll
            for (int j = 0; j < NB; ++j) m = fmaxf(m, fabsf(acc[i][j][e]));
#pragma unroll
            for (int s = 1; s < 32; s <<= 1) m = fmaxf(m, __shfl_xor(m, s));
            const float scale = m > 0.f ? __fdiv_rn(m, 448.0f) : 1.0f;
            // x / scale rounded to nearest: one correctly rounded reciprocal per row, then per
            // element q = x r and one correction with the exact residual x - q scale (Markstein)
            const float r = __fdiv_rn(1.0f, scale);
            const int64_t row = m0 + 64 * wm + 32 * i + 8 * (e >> 2) + 4 * hb + (e & 3);
            float y[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const float x = acc[i][j][e];
                const float q = x * r;
                y[j] = fmaf(fmaf(-q, scale, x), r, q);
            }
            // E4M3FN codes (nearest, ties to even) of columns 32 j + n, byte j of pk
            uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
            if constexpr (NB == 4) pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], (int)pk, true);
            if (row < a.T) {
                uint8_t* orow = out + row * a.stride;
#pragma unroll
                for (int j = 0; j < NB; ++j) orow[32 * j + n] = (uint8_t)(pk >> (8 * j));
            }
            if (row < a.T && n == 0) sout[row] = scale;
        }
}

hipError_t launch_bridge_fp8(const BridgeFp8Args& a, hipStream_t s) {
    ProfScope ps("bridge_fp8", s);
    dim3 grid((unsigned)(((a.T + kB8M - 1) / kB8M) * a.L));
    if (a.d == 128) bridge_fp8_kernel<128><<<grid, kB8Threads, 0, s>>>(a);
    else bridge_fp8_kernel<64><<<grid, kB8Threads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace hs2
