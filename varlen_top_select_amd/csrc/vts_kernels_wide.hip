// vts_kernels_wide.hip -- launches of the top-k kernels for top_k above 2048
// (up to 16384): candidate lists that outgrow the registers are kept in LDS
// and the workspace and selected from there.  A code object of its own, so
// the kernels for smaller top_k keep their code.
#include "vts_topk.hpp"

namespace vts {

template <int DT, class Policy>
static hipError_t launch_dt(const Params& p, hipStream_t stream) {
    const uint32_t grid = (uint32_t)p.units_per_xcd * 8u;
    hipLaunchKernelGGL((topk_kernel<DT, Policy, true>), dim3(grid), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_varlen_wide(int dtype, const Params& p, hipStream_t stream) {
    switch (dtype) {
        case F32: return launch_dt<F32, VarlenPolicy>(p, stream);
        case BF16: return launch_dt<BF16, VarlenPolicy>(p, stream);
        case F16: return launch_dt<F16, VarlenPolicy>(p, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_transform_wide(int dtype, const Params& p, hipStream_t stream) {
    switch (dtype) {
        case F32: return launch_dt<F32, PagePolicy>(p, stream);
        case BF16: return launch_dt<BF16, PagePolicy>(p, stream);
        case F16: return launch_dt<F16, PagePolicy>(p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace vts
