// Device code of the score pass: score_rows_dev.h (shared with the single-launch decode block).
#include "score_rows_dev.h"

namespace hs2 {

template <int D, int KV>
__global__ __launch_bounds__(256, 2) void score_rows_mfma_kernel(ScoreArgs a) {
    __shared__ ScoreLds S;
    score_rows_body<D, KV>(a, blockIdx.x, blockIdx.y, S);
}

// ---- launcher ------------------------------------------------------------------------------------
hipError_t launch_score_rows_mfma(const ScoreArgs& a, hipStream_t s) {
    ProfScope ps("score_rows_mfma", s);
    dim3 grid(a.B * a.Tq, a.nsplit);
    if (a.kv_dtype == HS2_FP8_E4M3) {
        if (a.d == 128) score_rows_mfma_kernel<128, HS2_FP8_E4M3><<<grid, 256, 0, s>>>(a);
        else score_rows_mfma_kernel<64, HS2_FP8_E4M3><<<grid, 256, 0, s>>>(a);
    } else {
        if (a.d == 128) score_rows_mfma_kernel<128, HS2_BF16><<<grid, 256, 0, s>>>(a);
        else score_rows_mfma_kernel<64, HS2_BF16><<<grid, 256, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace hs2
