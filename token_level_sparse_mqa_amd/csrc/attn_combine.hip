// Device code of the split merge: attn_combine_dev.h (shared with the single-launch decode block).
#include "attn_combine_dev.h"

namespace hs2 {

// Many splits (long rows): grid (row, head, D/16), 256 threads = 16 dims x 16 split lanes.
template <int D>
__global__ __launch_bounds__(256) void attn_split_combine_wide_kernel(AttnArgs a) {
    __shared__ CombineWideLds S;
    combine_wide_body<D>(a, blockIdx.x, blockIdx.y, blockIdx.z, S);
}

// Few splits: one workgroup per (row, head), one thread per dv.
template <int D>
__global__ __launch_bounds__(D) void attn_split_combine_kernel(AttnArgs a) {
    combine_narrow_body<D>(a, blockIdx.x, blockIdx.y);
}

// ---- launcher ------------------------------------------------------------------------------------
hipError_t launch_attn_split_combine(const AttnArgs& a, const char* name, hipStream_t s) {
    ProfScope ps(name, s);
    if (a.nsplit > kCombineNarrowMax) {
        dim3 grid(a.B * a.Tq * (a.nlayer > 1 ? a.nlayer : 1), a.H, a.d / 16);
        if (a.d == 128) attn_split_combine_wide_kernel<128><<<grid, 256, 0, s>>>(a);
        else attn_split_combine_wide_kernel<64><<<grid, 256, 0, s>>>(a);
    } else {
        dim3 grid(a.B * a.Tq * (a.nlayer > 1 ? a.nlayer : 1), a.H);
        if (a.d == 128) attn_split_combine_kernel<128><<<grid, 128, 0, s>>>(a);
        else attn_split_combine_kernel<64><<<grid, 64, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace hs2
