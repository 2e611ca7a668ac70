// vts_probe.hip -- two plain streaming kernels used only to calibrate
// measurements of the top-k kernels on the same device:
//   vts_probe_read  reads a buffer once with 16-byte non-temporal loads (the
//                   achievable read-bandwidth ceiling for the same bytes; the
//                   hint, which the top-k stream uses too, is worth about 12 %);
//   vts_probe_copy  copies a buffer with 16-byte loads and stores (a kernel of
//                   known traffic, to scale the FETCH_SIZE / WRITE_SIZE counters).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/vts_probe.h"

namespace {

constexpr int PT = 256;
constexpr int PU = 8;

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
#define GL __attribute__((address_space(1)))

__global__ void __launch_bounds__(PT) read_kernel(const v4u* __restrict__ p_, size_t nvec,
                                                  uint32_t* __restrict__ sink) {
    const GL v4u* p = (const GL v4u*)p_;
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * PT * PU;
    for (size_t base = (size_t)blockIdx.x * PT * PU + threadIdx.x; base < nvec; base += stride) {
        v4u v[PU];
#pragma unroll
        for (int u = 0; u < PU; ++u) {
            const size_t i = base + (size_t)u * PT;
            v[u] = i < nvec ? __builtin_nontemporal_load(p + i) : v4u{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < PU; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) ((GL uint32_t*)sink)[blockIdx.x] = acc;  // keeps the loads alive
}

__global__ void __launch_bounds__(PT) copy_kernel(v4u* __restrict__ dst_, const v4u* __restrict__ src_,
                                                  size_t nvec) {
    GL v4u* dst = (GL v4u*)dst_;
    const GL v4u* src = (const GL v4u*)src_;
    const size_t stride = (size_t)gridDim.x * PT;
    for (size_t i = (size_t)blockIdx.x * PT + threadIdx.x; i < nvec; i += stride) dst[i] = src[i];
}

int grid_for(size_t nvec, int per_block) {
    size_t g = (nvec + per_block - 1) / per_block;
    const size_t cap = 256 * 16;  // 16 workgroups per CU of an MI355X
    if (g > cap) g = cap;
    if (g < 1) g = 1;
    return (int)g;
}

}  // namespace

extern "C" {

int vts_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink || ((uintptr_t)buf % 16) || (bytes % 16)) return -1;
    const size_t nvec = bytes / 16;
    hipLaunchKernelGGL(read_kernel, dim3(grid_for(nvec, PT * PU)), dim3(PT), 0,
                       static_cast<hipStream_t>(stream), static_cast<const v4u*>(buf), nvec, sink);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int vts_probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (!dst || !src || ((uintptr_t)dst % 16) || ((uintptr_t)src % 16) || (bytes % 16)) return -1;
    const size_t nvec = bytes / 16;
    hipLaunchKernelGGL(copy_kernel, dim3(grid_for(nvec, PT)), dim3(PT), 0,
                       static_cast<hipStream_t>(stream), static_cast<v4u*>(dst),
                       static_cast<const v4u*>(src), nvec);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
