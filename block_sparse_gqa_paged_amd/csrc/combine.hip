// Log-sum-exp merge of (o, m, l) partials for gfx950: the standalone merge launch (the per-wave
// loop and the operation it computes are in combine_rows.h). The pass streams the partial
// vectors once: HBM-bound.
#include "combine_rows.h"

namespace pa {
namespace {

template <int D, int R>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a, int mode) {
    combine_rows<D, R>(a, mode, (blockIdx.x * blockDim.x + threadIdx.x) >> 6,
                       (gridDim.x * blockDim.x) >> 6);
}

}  // namespace

// mode: group_ptr given -> CSR; items given -> planner list; else uniform splits.
pa_status launch_combine(const CombineArgs &a, int max_groups, hipStream_t stream) {
    LaunchScope scope("combine", stream);
    const int mode = a.items ? 2 : (a.group_ptr ? 1 : 0);
    if (max_groups <= 0) return PA_OK;
    const long long waves = combine_waves(max_groups, a.lanes, a.D);
    const int grid = (int)((waves + 3) / 4);
    const int R = combine_r(a.lanes, a.D);
    switch (a.D * 4 + R) {
        case 64 * 4 + 1: scope.launch(combine_kernel<64, 1>, dim3(grid), dim3(256), 0, a, mode); break;
        case 64 * 4 + 2: scope.launch(combine_kernel<64, 2>, dim3(grid), dim3(256), 0, a, mode); break;
        case 128 * 4 + 1:
            scope.launch(combine_kernel<128, 1>, dim3(grid), dim3(256), 0, a, mode);
            break;
        case 128 * 4 + 2:
            scope.launch(combine_kernel<128, 2>, dim3(grid), dim3(256), 0, a, mode);
            break;
        case 256 * 4 + 1:
            scope.launch(combine_kernel<256, 1>, dim3(grid), dim3(256), 0, a, mode);
            break;
        case 256 * 4 + 2:
            scope.launch(combine_kernel<256, 2>, dim3(grid), dim3(256), 0, a, mode);
            break;
        default:
            return PA_ERR_UNSUPPORTED;
    }
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa
