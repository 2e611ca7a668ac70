// Exercise of the C ABI's host side (argument checks, plans, workspace sizes,
// status strings, per-thread switches) under AddressSanitizer and
// UndefinedBehaviorSanitizer on the host side (the kernels are not built: the
// launch entry points below stand in for them and launch nothing).  Every
// call uses fake device pointers; calls that pass every host check stop at the
// device query (no GPU) or at a stand-in launch.  Exits non-zero on a status
// other than the expected one.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <thread>

#include "../../include/vts.h"

namespace vts {
struct Params;
hipError_t launch_varlen(int, const Params&, hipStream_t) { return hipSuccess; }
hipError_t launch_transform(int, const Params&, hipStream_t) { return hipSuccess; }
hipError_t launch_row_batch(const int32_t*, int32_t, int32_t, int32_t*, hipStream_t) {
    return hipSuccess;
}
hipError_t launch_zero(uint32_t*, size_t, hipStream_t) { return hipSuccess; }
}  // namespace vts

static int bad = 0;
static void expect(const char* what, int got, int want) {
    if (got != want) {
        fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
        ++bad;
    }
}

int main() {
    char* A = reinterpret_cast<char*>(0x10000000);  // never dereferenced on the host
    int32_t* I = reinterpret_cast<int32_t*>(A);
    const size_t big = (size_t)1 << 40;
    // varlen: every class of argument error
    expect("dtype", vts_topk_varlen(A, 3, 8, 4096, 4096, I, 512, 1, 1, 0, I, 0, A, big, 0), VTS_ERR_INVALID);
    expect("rows", vts_topk_varlen(A, 0, -1, 4096, 4096, I, 512, 1, 1, 0, I, 0, A, big, 0), VTS_ERR_INVALID);
    expect("stride", vts_topk_varlen(A, 0, 8, 4096, 100, I, 512, 1, 1, 0, I, 0, A, big, 0), VTS_ERR_INVALID);
    expect("k0", vts_topk_varlen(A, 0, 8, 4096, 4096, I, 0, 1, 1, 0, I, 0, A, big, 0), VTS_ERR_INVALID);
    expect("kbig", vts_topk_varlen(A, 0, 8, 4096, 4096, I, 16385, 1, 1, 0, I, 0, A, big, 0), VTS_ERR_UNSUPPORTED);
    expect("next_n", vts_topk_varlen(A, 0, 8, 4096, 4096, I, 512, 3, 1, 0, I, 0, A, big, 0), VTS_ERR_INVALID);
    expect("cr", vts_topk_varlen(A, 0, 8, 4096, 4096, I, 512, 1, 0, 0, I, 0, A, big, 0), VTS_ERR_INVALID);
    expect("out", vts_topk_varlen(A, 0, 8, 4096, 4096, I, 512, 1, 1, 0, I + 1, 0, A, big, 0), VTS_ERR_INVALID);
    expect("overlap", vts_topk_varlen(A, 0, 8, 4096, 4096, I, 512, 1, 1, 0, I, A + 4096, A, big, 0), VTS_ERR_INVALID);
    expect("ws", vts_topk_varlen(A, 0, 8, 4096, 4096, I, 512, 1, 1, 0, I, 0, A, 16, 0), VTS_ERR_WORKSPACE);
    expect("zero rows", vts_topk_varlen(0, 0, 0, 4096, 4096, 0, 512, 1, 1, 0, 0, 0, 0, 0, 0), VTS_OK);
    expect("ordered k", vts_topk_varlen_ordered(A, 0, 8, 4096, 4096, I, 2049, 1, 1, 0, I, 0, A, big, 0, 1), VTS_ERR_UNSUPPORTED);
    expect("tie", vts_topk_varlen_ordered(A, 0, 8, 4096, 4096, I, 512, 1, 1, 0, I, 0, A, big, 0, 3), VTS_ERR_INVALID);
    expect("noalloc size", vts_topk_varlen_noalloc(A, 0, 2048, 262144, 262144, I, 2048, 1, 1, 0, I, 0, 0), VTS_ERR_TOO_LARGE);
    // transforms
    expect("page size", vts_topk_page_table_transform(A, 2, 4, 1024, 1040, I, 0, I, 32, 32, 0, 0, 256, I, 0, A, big, 0), VTS_ERR_INVALID);
    expect("ptrs", vts_topk_page_table_transform(A, 2, 4, 1024, 1040, I, I, I, 32, 32, 0, 64, 256, I, 0, A, big, 0), VTS_ERR_INVALID);
    expect("raw overlap", vts_topk_page_table_transform(A, 2, 4, 1024, 1040, I, 0, I, 32, 32, 0, 64, 256, I, I + 256, A, big, 0), VTS_ERR_INVALID);
    expect("ragged", vts_topk_transform_ragged(A, 2, 4, 1024, 1040, 0, 0, I, 256, I, 0, A, big, 0), VTS_ERR_INVALID);
    expect("page1", vts_topk_transform_page1(A, 2, 4, 1024, 1040, I, 0, I, 32, 32, 0, 2, 256, I, 0, A, big, 0), VTS_ERR_INVALID);
    // valid calls: the host checks pass, the device query fails without a GPU
    const int dev = vts_topk_varlen(A, 0, 8, 4096, 4096, I, 512, 1, 1, 0, I, 0, A, big, 0);
    if (dev != VTS_ERR_HIP && dev != VTS_OK && dev != VTS_ERR_UNSUPPORTED) expect("valid call", dev, VTS_ERR_HIP);
    // workspace sizes over many shapes (pure functions), status strings
    for (int64_t r = 0; r < 5000; r += 37)
        for (int32_t k = 1; k <= 16384; k *= 3)
            if (vts_topk_varlen_workspace_bytes(r, 1 + r * 97, k, 0) < 256) expect("ws size", 0, 1);
    for (int st = -6; st <= 2; ++st)
        if (vts_status_string(st) == nullptr) expect("status string", st, 0);
    // per-thread switches
    std::thread t([] { vts_set_tuning(VTS_TUNE_NSPLIT, 1); });
    t.join();
    const size_t a = vts_topk_varlen_workspace_bytes(64, 163840, 2048, 0);
    vts_set_tuning(VTS_TUNE_NSPLIT, 1);
    const size_t b = vts_topk_varlen_workspace_bytes(64, 163840, 2048, 0);
    vts_set_tuning(VTS_TUNE_NSPLIT, 0);
    if (!(b < a)) expect("thread switch", 0, 1);
    if (bad) return 1;
    printf("host battery clean\n");
    return 0;
}
