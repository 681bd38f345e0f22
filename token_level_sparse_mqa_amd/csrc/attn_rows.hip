// Device code of the row kernel: attn_rows_dev.h (shared with the single-launch decode block).
#include "attn_rows_dev.h"

namespace hs2 {

// Two workgroups (eight waves) per CU, so while one wave waits on LDS or MFMA results the other
// computes; each wave keeps its next tile in flight in registers.
template <int D, int KV, bool LIST, bool REUSE>
__global__ __launch_bounds__(kRowWaves * 64, 2)
void attn_rows_mfma_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) RowLds<D> S;
    attn_rows_body<D, KV, LIST, REUSE>(a, blockIdx.x, blockIdx.y, S);
}

// ---- launcher ------------------------------------------------------------------------------------
template <bool LIST, bool REUSE>
void launch_rows(const AttnArgs& a, dim3 grid, hipStream_t s) {
    if (a.kv_dtype == HS2_FP8_E4M3) {
        if (a.d == 128) attn_rows_mfma_kernel<128, HS2_FP8_E4M3, LIST, REUSE><<<grid, kRowWaves * 64, 0, s>>>(a);
        else attn_rows_mfma_kernel<64, HS2_FP8_E4M3, LIST, REUSE><<<grid, kRowWaves * 64, 0, s>>>(a);
    } else {
        if (a.d == 128) attn_rows_mfma_kernel<128, HS2_BF16, LIST, REUSE><<<grid, kRowWaves * 64, 0, s>>>(a);
        else attn_rows_mfma_kernel<64, HS2_BF16, LIST, REUSE><<<grid, kRowWaves * 64, 0, s>>>(a);
    }
}

hipError_t launch_attn_rows_mfma(const AttnArgs& a, const char* name, hipStream_t s) {
    ProfScope ps(name, s);
    dim3 grid(a.B * a.Tq * (a.nlayer > 1 ? a.nlayer : 1), a.nsplit);
    // index lists of query chunks gather with cached loads, those of decode rows non-temporally
    if (a.list && a.Tq >= kPrefillMinTq) launch_rows<true, true>(a, grid, s);
    else if (a.list) launch_rows<true, false>(a, grid, s);
    else launch_rows<false, false>(a, grid, s);
    return hipGetLastError();
}

}  // namespace hs2
