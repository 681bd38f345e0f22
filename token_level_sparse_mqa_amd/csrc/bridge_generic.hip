// Generic KV-Bridge projection (VALU, fp32 accumulate): [K | V] = hidden . [Wk | Wv].
//
// KV Bridging (lynxflow blog, "Two-Level KV Sharing"; ainews page, mechanism paragraph):
// the cross-decoder full-attention layer's K/V are projections of self-decoder hidden
// states, with the layer's own projections.  Output rows are rounded once to bf16 (RNE).
#include "hs2_device.h"

namespace hs2 {

constexpr int kBgM = 64, kBgN = 64, kBgK = 32;

__global__ __launch_bounds__(256) void bridge_generic_kernel(BridgeArgs a) {
    __shared__ float hs[kBgM][kBgK + 1];
    __shared__ float ws[kBgK][kBgN + 4];
    const int64_t m0 = (int64_t)blockIdx.x * kBgM;
    const int n0 = blockIdx.y * kBgN;                  // column in [0, 2d)
    const int tid = threadIdx.x;
    const int tr = (tid >> 4) * 4, tc = (tid & 15) * 4;
    float acc[4][4] = {};
    const uint16_t* w = n0 < a.d ? a.wk : a.wv;
    const int wc0 = n0 < a.d ? n0 : n0 - a.d;
    for (int k0 = 0; k0 < a.D; k0 += kBgK) {
        for (int x = tid; x < kBgM * kBgK; x += 256) {
            const int i = x / kBgK, c = x % kBgK;
            const int64_t row = m0 + i;
            hs[i][c] = row < a.T ? bf16_to_f32(a.hidden[row * a.D + k0 + c]) : 0.f;
        }
        for (int x = tid; x < kBgK * kBgN; x += 256) {
            const int i = x / kBgN, c = x % kBgN;
            ws[i][c] = bf16_to_f32(w[(int64_t)(k0 + i) * a.d + wc0 + c]);
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < kBgK; ++kk) {
            float hv[4], wv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) { hv[u] = hs[tr + u][kk]; wv[u] = ws[kk][tc + u]; }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[u][v] += hv[u] * wv[v];
        }
        __syncthreads();
    }
    uint16_t* out = n0 < a.d ? a.k_out : a.v_out;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t row = m0 + tr + u;
        if (row >= a.T) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) out[row * a.stride + wc0 + tc + v] = f32_to_bf16_rne(acc[u][v]);
    }
}

hipError_t launch_bridge_generic(const BridgeArgs& a, hipStream_t s) {
    ProfScope ps("bridge_generic", s);
    dim3 grid((unsigned)((a.T + kBgM - 1) / kBgM), (2 * a.d) / kBgN);
    bridge_generic_kernel<<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace hs2
