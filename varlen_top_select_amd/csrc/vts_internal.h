// vts_internal.h -- kernel parameter block and launch entry points shared by
// the kernels (vts_kernels.hip) and the C ABI (vts_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vts {

// Candidate slots per workgroup in the workspace (Params::ws_slots, at most
// HI_SLOTS): they mirror the unit's candidate list (the first, on-chip slots
// are copied there only when a split row publishes them; later slots are
// where the list spills).
constexpr int HI_SLOTS = 8192;

// top_k of the kernels that hold a candidate list in registers; larger top_k
// (up to K_MAX) run the wide kernels, whose lists live in LDS and the
// workspace (2 * top_k rounded up to a power of two slots per unit).
constexpr int NARROW_K_MAX = 2048;
constexpr int K_MAX = 16384;

inline int32_t slots_for_k(int32_t k) {
    if (k <= NARROW_K_MAX) return HI_SLOTS;
    int32_t pw = 1;
    while (pw < k) pw <<= 1;
    return 2 * pw;
}

// Compute units of an MI355X: 8 XCDs of 32.  Block b of a launch goes to XCD
// b % 8, and there the k-th block (b = 8k + x) to compute unit k % 32 while
// the first blocks fill the device, so blocks k, k + 32, k + 64, ... of an
// XCD share a compute unit.
constexpr int BALANCE_XCDS = 8;
constexpr int BALANCE_CUS_PER_XCD = 32;
constexpr int BALANCE_CUS = BALANCE_XCDS * BALANCE_CUS_PER_XCD;

// Output order: any (fastest), or the deterministic mode: the ties at the
// k-th value taken at the smallest (ORDER_SMALL) or largest (ORDER_LARGE)
// columns, listed in canonical order (value descending, column ascending)
// unless ORDER_NOSORT is added (the same set, in no particular order).
constexpr int ORDER_ANY = 0, ORDER_SMALL = 1, ORDER_LARGE = 2, ORDER_NOSORT = 4;

struct Params {
    // score rows
    const void* x;
    int64_t row_stride;  // elements
    int64_t width;
    int32_t num_rows;
    int32_t k;
    // topk_varlen rows
    const int32_t* seq_lens;
    int32_t next_n;
    int32_t cr;
    const int32_t* pre_idx;  // the hint (request-major, k per request), or null
    int32_t hint_rung;       // 1: bound the safe rung by the hint rung as well (diagnostic)
    // page-transform rows
    const int32_t* lengths;
    const int32_t* row_starts;
    const int32_t* pt;
    int64_t pt_stride;
    int64_t pt_width;
    const int32_t* ptrs;
    int32_t page_size;
    const int32_t* offsets;  // ragged transform: per-row index offset (null: page table)
    const int32_t* row_batch;  // page-size-1 transform: each row's request (page-table row), or -1
    // outputs
    int32_t* out_idx;  // topk_varlen: indices; transform: translated `out`
    void* out_vals;    // topk_varlen values or null
    int32_t* out_raw;  // transform raw indices or null
    // plan
    int32_t nsplit;     // workgroups per row (1..MAX_SPLIT)
    int32_t min_chunk;  // a row gets ceil(n / min_chunk) workgroups, at most nsplit
    int32_t num_units;  // num_rows * nsplit
    int32_t units_per_xcd;
    int32_t balance;    // 1: rows are assigned to workgroups by length (see balanced_row)
    int32_t lds_cap;    // on-chip candidate slots used before spilling (<= CAP)
    int32_t hi_cap;     // candidate slots in all (<= ws_slots) before re-filtering
    int32_t ws_slots;   // workspace slots per unit (the stride of ws_key / ws_idx)
    int32_t force_path;
    float sigma;        // margin of the safe rung, in standard deviations
    float sigma2;       // margin of the likely rung (<= sigma)
    // workspace
    uint32_t* ws_stats;
    uint32_t* ws_ticket;
    uint32_t* ws_count;     // candidates (keys >= the safe rung) per unit
    uint32_t* ws_count_up;  // of which keys >= the likely rung, per unit
    uint32_t* ws_key;
    uint32_t* ws_idx;
    int32_t order;  // ORDER_ANY, or ORDER_SMALL / ORDER_LARGE (+ ORDER_NOSORT)
    int32_t helpers;     // balanced placement of 2 * BALANCE_CUS rows cut into length-balanced units
    int32_t split_cols;  // (helpers) the shortest unit, in columns
#ifdef VTS_PHASE_STAMPS
    uint64_t* stamps;  // phase-timing build: VTS_STAMPS_PER_UNIT stamps per unit, or null
#endif
};

#ifdef VTS_PHASE_STAMPS
constexpr int VTS_STAMPS_PER_UNIT = 16;
#endif

enum { FORCE_NONE = 0, FORCE_CAREFUL = 1, FORCE_FALLBACK = 2 };

// Workspace layout (bytes from the base): stats, tickets, counts, keys, indices.
struct WsLayout {
    size_t stats, ticket, count, count_up, key, idx, batch, total;
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

inline WsLayout ws_layout(int64_t num_rows, int32_t nsplit, int32_t slots = HI_SLOTS) {
    WsLayout L;
    const size_t units = (size_t)num_rows * (size_t)nsplit;
    L.stats = 0;
    L.ticket = 256;
    L.count = L.ticket + align256((size_t)num_rows * 4);
    L.count_up = L.count + align256(units * 4);
    L.key = L.count_up + align256(units * 4);
    L.idx = L.key + align256(units * (size_t)slots * 4);
    L.batch = L.idx + align256(units * (size_t)slots * 4);  // one int32 per row (request map)
    L.total = L.batch + align256((size_t)num_rows * 4);
    return L;
}

hipError_t launch_varlen(int dtype, const Params& p, hipStream_t stream);
hipError_t launch_transform(int dtype, const Params& p, hipStream_t stream);
hipError_t launch_varlen_ordered(int dtype, const Params& p, hipStream_t stream);
hipError_t launch_varlen_wide(int dtype, const Params& p, hipStream_t stream);
hipError_t launch_varlen_hint(int dtype, const Params& p, hipStream_t stream);
hipError_t launch_transform_wide(int dtype, const Params& p, hipStream_t stream);
// Zeroes `words` 32-bit words at `p` (a kernel, so it can sit in a captured graph).
hipError_t launch_zero(uint32_t* p, size_t words, hipStream_t stream);
hipError_t launch_transform_ordered(int dtype, const Params& p, hipStream_t stream);
// Writes each row's request b (cu_seqlens[b] <= row < cu_seqlens[b + 1]) or -1.
hipError_t launch_row_batch(const int32_t* cu_seqlens, int32_t num_batches, int32_t num_rows,
                            int32_t* row_batch, hipStream_t stream);

}  // namespace vts
