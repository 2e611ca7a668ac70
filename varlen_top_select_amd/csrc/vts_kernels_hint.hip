// vts_kernels_hint.hip -- launches of the varlen top-k kernels for calls that
// pass the previous step's selection (pre_idx, top_k <= 2048): their safe
// rung is the larger of the sampled rung and the hint rung.  A code object of
// its own, so the hint-free kernels keep their code and registers.
#include "vts_topk.hpp"

namespace vts {

template <int DT>
static hipError_t launch_dt(const Params& p, hipStream_t stream) {
    const uint32_t grid = (uint32_t)p.units_per_xcd * 8u;
    hipLaunchKernelGGL((topk_kernel<DT, VarlenPolicy, false, true>), dim3(grid), dim3(NT), 0,
                       stream, p);
    return hipGetLastError();
}

hipError_t launch_varlen_hint(int dtype, const Params& p, hipStream_t stream) {
    switch (dtype) {
        case F32: return launch_dt<F32>(p, stream);
        case BF16: return launch_dt<BF16>(p, stream);
        case F16: return launch_dt<F16>(p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace vts
