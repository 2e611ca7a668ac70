// vts_kernels_ordered.hip -- launches of the deterministic-mode kernels
// (canonical keys, SMALL / LARGE tie-break, canonical order), built as a code
// object of their own so they do not move the other kernels' code.
#include "vts_topk.hpp"

namespace vts {

template <int DT, class Policy>
static hipError_t launch_dt(const Params& p, hipStream_t stream) {
    const uint32_t grid = (uint32_t)p.units_per_xcd * 8u;
    hipLaunchKernelGGL((topk_kernel<DT, Policy>), dim3(grid), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_varlen_ordered(int dtype, const Params& p, hipStream_t stream) {
    switch (dtype) {
        case F32: return launch_dt<F32, OrderedVarlenPolicy>(p, stream);
        case BF16: return launch_dt<BF16, OrderedVarlenPolicy>(p, stream);
        case F16: return launch_dt<F16, OrderedVarlenPolicy>(p, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_transform_ordered(int dtype, const Params& p, hipStream_t stream) {
    switch (dtype) {
        case F32: return launch_dt<F32, OrderedPagePolicy>(p, stream);
        case BF16: return launch_dt<BF16, OrderedPagePolicy>(p, stream);
        case F16: return launch_dt<F16, OrderedPagePolicy>(p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace vts
