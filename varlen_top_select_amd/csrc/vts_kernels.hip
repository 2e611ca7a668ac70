// vts_kernels.hip -- launches of the top-k kernels (any output order) and of
// the row-to-request map of the page-size-1 transform.  The kernels of the
// deterministic mode are in vts_kernels_ordered.hip, a code object of its own.
#include "vts_topk.hpp"

namespace vts {

template <int DT, class Policy>
static hipError_t launch_dt(const Params& p, hipStream_t stream) {
    const uint32_t grid = (uint32_t)p.units_per_xcd * 8u;
    hipLaunchKernelGGL((topk_kernel<DT, Policy>), dim3(grid), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_varlen(int dtype, const Params& p, hipStream_t stream) {
    if (p.order != ORDER_ANY) return launch_varlen_ordered(dtype, p, stream);
    if (p.k > NARROW_K_MAX) return launch_varlen_wide(dtype, p, stream);
    if (p.pre_idx && p.hint_rung) return launch_varlen_hint(dtype, p, stream);
    switch (dtype) {
        case F32: return launch_dt<F32, VarlenPolicy>(p, stream);
        case BF16: return launch_dt<BF16, VarlenPolicy>(p, stream);
        case F16: return launch_dt<F16, VarlenPolicy>(p, stream);
    }
    return hipErrorInvalidValue;
}

// Row -> request map of the page-size-1 transform: row r belongs to the request
// b with cu_seqlens[b] <= r < cu_seqlens[b + 1] (SGLang TopK_Ops,
// `cu_seqlens_q`), found by binary search over the non-decreasing offsets; a
// row outside [cu_seqlens[0], cu_seqlens[num_batches]) gets -1.
__global__ void __launch_bounds__(NT) row_batch_kernel(const int32_t* cu, int32_t nb, int32_t rows,
                                                       int32_t* row_batch) {
    const int32_t r = (int32_t)(blockIdx.x * NT + threadIdx.x);
    if (r >= rows) return;
    int32_t b = -1;
    if (nb > 0 && gload(cu) <= r && r < gload(cu + nb)) {
        int32_t lo = 0, hi = nb;  // cu[lo] <= r < cu[hi]
        while (hi - lo > 1) {
            const int32_t mid = lo + (hi - lo) / 2;
            if (gload(cu + mid) <= r) lo = mid; else hi = mid;
        }
        b = lo;
    }
    gstore(row_batch + r, b);
}

hipError_t launch_row_batch(const int32_t* cu_seqlens, int32_t num_batches, int32_t num_rows,
                            int32_t* row_batch, hipStream_t stream) {
    const uint32_t grid = ((uint32_t)num_rows + NT - 1) / NT;
    hipLaunchKernelGGL(row_batch_kernel, dim3(grid), dim3(NT), 0, stream, cu_seqlens, num_batches,
                       num_rows, row_batch);
    return hipGetLastError();
}

__global__ void __launch_bounds__(NT) zero_kernel(uint32_t* p, uint32_t words) {
    const uint32_t i = blockIdx.x * NT + threadIdx.x;
    if (i < words) gstore(p + i, 0u);
}

hipError_t launch_zero(uint32_t* p, size_t words, hipStream_t stream) {
    if (words == 0) return hipSuccess;
    const uint32_t grid = (uint32_t)((words + NT - 1) / NT);
    hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(NT), 0, stream, p, (uint32_t)words);
    return hipGetLastError();
}

hipError_t launch_transform(int dtype, const Params& p, hipStream_t stream) {
    if (p.order != ORDER_ANY) return launch_transform_ordered(dtype, p, stream);
    if (p.k > NARROW_K_MAX) return launch_transform_wide(dtype, p, stream);
    switch (dtype) {
        case F32: return launch_dt<F32, PagePolicy>(p, stream);
        case BF16: return launch_dt<BF16, PagePolicy>(p, stream);
        case F16: return launch_dt<F16, PagePolicy>(p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace vts
