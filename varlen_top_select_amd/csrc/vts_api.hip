// vts_api.hip -- C ABI of the top-k library: argument checks (host only, before
// any HIP call), the launch plan (a pure function of the static shape, so a
// call can be captured in a HIP graph), workspace sizing and the launch.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/vts.h"
#include "vts_device.hpp"
#include "vts_internal.h"

namespace {

using namespace vts;

// Units of work per launch the plan aims for: one workgroup per compute unit of
// an MI355X (256 CUs).  Rows are split only while there are fewer rows than
// that: every unit of a split row pays the sample and rung start and the row
// pays a merge, which costs more than a partly idle launch (measured: 256 fp16
// rows of 65536 run faster unsplit, 64 fp32 rows of 163840 fastest in four).
// A fixed constant keeps the plan -- and the workspace size -- independent of
// the device query.
constexpr int64_t TARGET_UNITS = 256;
// A row gets at most one workgroup per MIN_CHUNK valid columns: below about
// 32K columns a split's fixed costs (its own sample and the merge) outweigh
// the shorter stream (measured on the five benchmark shapes).
constexpr int32_t MIN_CHUNK = 32768;

// Diagnostic and test switches (vts_set_tuning).
struct Tuning {
    int32_t nsplit = 0;
    int32_t force_path = 0;
    int32_t lds_slots = 0;
    int32_t spill_slots = 0;
    int32_t sigma_tenths = 0;
    int32_t min_chunk = 0;
    int32_t likely_tenths = 0;
    int32_t no_balance = 0;
    int32_t hint_rung = 0;
};
// per calling thread: a switch set for a test or a measurement changes only
// the calls (and workspace-size queries) of the thread that set it
thread_local Tuning g_tune;

#ifdef VTS_PHASE_STAMPS
uint64_t* g_stamps = nullptr;  // phase-timing build: where the next launches stamp
#endif

size_t itemsize(int32_t dtype) { return dtype == VTS_F32 ? 4 : 2; }

// With the length-balanced placement of 2 * BALANCE_CUS rows (two per compute
// unit), the launch has twice as many workgroups and every row is cut into
// units of about the batch's columns per compute unit (placed_unit in the
// kernel): one workgroup's stream is capped by the memory requests its
// compute unit keeps in flight (~20 GB/s), so a row far longer than the mean
// would otherwise finish long after the rest.  A unit is at least
// MIN_UNIT_BYTES long: a split pays a sample per unit and a merge (DSv4 MTP,
// cold: 29.0 us at 128 KB, 30.8 at 96, 29.9 at 192, 31.9 at 64).  The rows
// are known only on the device, which decides per row; the plan reserves the
// workgroups and the workspace.
constexpr int64_t MIN_UNIT_BYTES = 128 * 1024;

int32_t split_cols(int32_t dtype) { return (int32_t)(MIN_UNIT_BYTES / (int64_t)itemsize(dtype)); }

bool helpers_apply(int64_t num_rows, int64_t width, int32_t dtype) {
    return num_rows == 2 * BALANCE_CUS && width >= split_cols(dtype) && g_tune.no_balance == 0;
}

int32_t plan_nsplit(int64_t num_rows, int64_t width, int32_t dtype) {
    if (g_tune.nsplit > 0) return g_tune.nsplit;
    if (num_rows <= 0) return 1;
    if (helpers_apply(num_rows, width, dtype)) return 2;
    int64_t ns = (TARGET_UNITS + num_rows - 1) / num_rows;
    const int64_t by_width = (width + MIN_CHUNK - 1) / MIN_CHUNK;
    if (ns > by_width) ns = by_width;
    if (ns > MAX_SPLIT) ns = MAX_SPLIT;
    if (ns < 1) ns = 1;
    return (int32_t)ns;
}

size_t workspace_bytes(int64_t num_rows, int64_t width, int32_t top_k, int32_t dtype) {
    if (num_rows <= 0) return 256;
    return ws_layout(num_rows, plan_nsplit(num_rows, width, dtype), slots_for_k(top_k)).total;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// Common checks of the score-row arguments.
int check_rows(const void* x, int32_t dtype, int64_t num_rows, int64_t width, int64_t row_stride,
               int32_t top_k) {
    if (dtype != VTS_F32 && dtype != VTS_BF16 && dtype != VTS_F16) return VTS_ERR_INVALID;
    if (num_rows < 0 || width < 1 || row_stride < width) return VTS_ERR_INVALID;
    if (top_k < 1) return VTS_ERR_INVALID;
    if (top_k > K_MAX) return VTS_ERR_UNSUPPORTED;
    if (width > INT32_MAX || num_rows > (int64_t)INT32_MAX / MAX_SPLIT) return VTS_ERR_UNSUPPORTED;
    // a row is streamed with 32-bit byte offsets
    if (width * (int64_t)itemsize(dtype) > (int64_t)INT32_MAX) return VTS_ERR_UNSUPPORTED;
    if (num_rows > 0 && (x == nullptr || !aligned(x, itemsize(dtype)))) return VTS_ERR_INVALID;
    return VTS_OK;
}

int check_workspace(void* ws, size_t bytes, int64_t num_rows, int64_t width, int32_t top_k,
                    int32_t dtype) {
    if (ws == nullptr || !aligned(ws, 16)) return VTS_ERR_WORKSPACE;
    if (bytes < workspace_bytes(num_rows, width, top_k, dtype)) return VTS_ERR_WORKSPACE;
    return VTS_OK;
}

// The device that work on `stream` runs on (the current device for the null
// stream), checked to be a gfx950, and its compute units; cached per device.
int check_device(void* stream, int* dev_out = nullptr, int* cus_out = nullptr) {
    static std::mutex mu;
    static int known[64];  // 0 unknown, 1 gfx950, 2 other
    static int cus[64];
    int dev = 0;
    if (stream == nullptr) {
        if (hipGetDevice(&dev) != hipSuccess) return VTS_ERR_HIP;
    } else {
        hipDevice_t d;
        if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &d) != hipSuccess)
            return VTS_ERR_HIP;
        dev = (int)d;
    }
    if (dev < 0 || dev >= 64) return VTS_ERR_UNSUPPORTED;
    if (dev_out) *dev_out = dev;
    std::lock_guard<std::mutex> lock(mu);
    if (known[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return VTS_ERR_HIP;
        known[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        cus[dev] = prop.multiProcessorCount;
    }
    if (cus_out) *cus_out = cus[dev];
    return known[dev] == 1 ? VTS_OK : VTS_ERR_UNSUPPORTED;
}

// Device scratch of vts_topk_varlen_noalloc, for callers that cannot
// allocate: one array per device, held by the loaded library until the
// process ends.  Host code never names it except in hipGetSymbolAddress, which
// gives each device's own address (scratch_of); those addresses are what the
// launches take.
constexpr size_t SCRATCH_BYTES = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

// The address of `scratch` on device `dev`, looked up once per device with
// that device current.
int scratch_of(int dev, void** out) {
    static std::mutex mu;
    static void* addr[64];
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess) return VTS_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return VTS_ERR_HIP;
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return VTS_ERR_HIP;
        if (e != hipSuccess || ptr == nullptr) return VTS_ERR_HIP;
        addr[dev] = ptr;
    }
    *out = addr[dev];
    return VTS_OK;
}

// Candidate slots per unit that let the workspace of this shape fit the
// scratch array (at most HI_SLOTS, in steps of 64), or 0 when even CAP slots
// per unit -- what a split row's units publish -- do not fit.
int32_t scratch_slots(int64_t num_rows, int64_t width, int32_t top_k, int32_t dtype) {
    const int32_t ns = plan_nsplit(num_rows, width, dtype);
    if (top_k > NARROW_K_MAX) {  // wide lists need all their slots
        const int32_t slots = slots_for_k(top_k);
        return ws_layout(num_rows, ns, slots).total <= SCRATCH_BYTES ? slots : 0;
    }
    for (int32_t slots = HI_SLOTS; slots >= CAP; slots -= 64)
        if (ws_layout(num_rows, ns, slots).total <= SCRATCH_BYTES) return slots;
    return 0;
}

// The launch plan and the workspace pointers; `slots` candidate slots per
// unit in the workspace (>= CAP whenever a row is split: a split row's units
// publish their on-chip lists there).
// `cus`: the device's compute units.  The length-balanced placement (and its
// units) assumes the dispatch order of 8 XCDs of 32 compute units
// (BALANCE_CUS); on any other device the rows run in order, one unit each
// where the plan reserved two (the workspace, sized from the shape alone, is
// then larger than needed).
void fill_plan(Params& p, int64_t num_rows, int64_t width, void* ws, int32_t slots, int32_t dtype,
               int cus) {
    const bool placed = cus == BALANCE_CUS && g_tune.no_balance == 0;
    int32_t ns = plan_nsplit(num_rows, width, dtype);
    const bool helpers = ns == 2 && g_tune.nsplit == 0 && helpers_apply(num_rows, width, dtype);
    if (helpers && !placed) ns = 1;
    const WsLayout L = ws_layout(num_rows, ns, slots);
    char* w = static_cast<char*>(ws);
    p.nsplit = ns;
    p.min_chunk = g_tune.min_chunk > 0 ? g_tune.min_chunk : MIN_CHUNK;
    p.num_units = (int32_t)(num_rows * ns);
    p.units_per_xcd = (p.num_units + 7) / 8;
    // length-balanced row placement: one workgroup per row, whole slots on all
    // 256 CUs (2..4 rows per CU, all resident at once)
    p.helpers = helpers && placed ? 1 : 0;
    p.split_cols = g_tune.min_chunk > 0 ? g_tune.min_chunk : split_cols(dtype);
    p.balance = ((ns == 1 && num_rows % BALANCE_CUS == 0 && num_rows >= 2 * BALANCE_CUS &&
                  num_rows <= 4 * BALANCE_CUS && placed) || p.helpers)
                    ? 1 : 0;
    p.lds_cap = g_tune.lds_slots > 0 ? g_tune.lds_slots : CAP;
    p.hi_cap = slots;
    if (g_tune.spill_slots > 0) p.hi_cap = g_tune.spill_slots;
    if (p.hi_cap > slots) p.hi_cap = slots;
    if (p.hi_cap < p.lds_cap) p.hi_cap = p.lds_cap;
    p.ws_slots = slots;
    p.force_path = g_tune.force_path;
    p.sigma = (g_tune.sigma_tenths > 0 ? g_tune.sigma_tenths : 50) / 10.0f;
    p.sigma2 = (g_tune.likely_tenths > 0 ? g_tune.likely_tenths : 20) / 10.0f;
    if (p.sigma2 > p.sigma) p.sigma2 = p.sigma;
    p.ws_stats = reinterpret_cast<uint32_t*>(w + L.stats);
    p.ws_ticket = reinterpret_cast<uint32_t*>(w + L.ticket);
    p.ws_count = reinterpret_cast<uint32_t*>(w + L.count);
    p.ws_count_up = reinterpret_cast<uint32_t*>(w + L.count_up);
    p.ws_key = reinterpret_cast<uint32_t*>(w + L.key);
    p.ws_idx = reinterpret_cast<uint32_t*>(w + L.idx);
#ifdef VTS_PHASE_STAMPS
    p.stamps = g_stamps;
#endif
}

// VTS_LOG=1 in the environment (read once): every call prints the plan it
// launches to stderr, one line.  Diagnostics only; results never depend on it.
bool log_on() {
    static const bool on = [] {
        const char* v = getenv("VTS_LOG");
        return v != nullptr && v[0] != '\0' && strcmp(v, "0") != 0;
    }();
    return on;
}

void log_plan(const char* entry, const Params& p, int32_t dtype, int64_t width, int cus) {
    if (!log_on()) return;
    static const char* const dts[] = {"f32", "bf16", "f16"};
    const char* kind = p.order != ORDER_ANY ? "ordered"
                       : p.k > NARROW_K_MAX ? "wide"
                       : (p.pre_idx && p.hint_rung) ? "hinted"
                       : "any-order";
    fprintf(stderr,
            "[vts] %s: rows %d width %lld top_k %d %s | kernels %s | units %d (%d per row%s) | "
            "placement %s | order %d | workspace slots %d per unit | device CUs %d\n",
            entry, p.num_rows, (long long)width, p.k, dtype >= 0 && dtype < 3 ? dts[dtype] : "?",
            kind, p.num_units, p.nsplit,
            p.helpers ? ", rows cut into length-balanced units" : "",
            p.balance ? "length-balanced" : "in row order", p.order, p.ws_slots, cus);
}

// tie_break argument -> internal order (false: invalid)
bool order_of(int32_t tie_break, int32_t* order) {
    const int32_t tb = tie_break & ~VTS_TIE_UNSORTED;
    if (tb != VTS_TIE_SMALL && tb != VTS_TIE_LARGE) return false;
    *order = (tb == VTS_TIE_SMALL ? ORDER_SMALL : ORDER_LARGE) |
             ((tie_break & VTS_TIE_UNSORTED) ? ORDER_NOSORT : 0);
    return true;
}

}  // namespace

extern "C" {

size_t vts_topk_varlen_workspace_bytes(int64_t num_rows, int64_t width, int32_t top_k,
                                       int32_t dtype) {
    return workspace_bytes(num_rows, width, top_k, dtype);
}

size_t vts_page_transform_workspace_bytes(int64_t num_rows, int64_t width, int32_t top_k,
                                          int32_t dtype) {
    return workspace_bytes(num_rows, width, top_k, dtype);
}

int vts_workspace_init(void* workspace, size_t bytes, void* stream) {
    if (workspace == nullptr) return VTS_ERR_WORKSPACE;
    if (hipMemsetAsync(workspace, 0, bytes, static_cast<hipStream_t>(stream)) != hipSuccess)
        return VTS_ERR_HIP;
    return VTS_OK;
}

// use_scratch: the device's scratch array instead of the caller's workspace
// (vts_topk_varlen_noalloc)
static int topk_varlen_impl(const void* logits, int32_t dtype, int64_t num_rows, int64_t width,
                            int64_t row_stride, const int32_t* seq_lens, int32_t top_k,
                            int32_t next_n, int32_t compress_ratio, const int32_t* pre_idx,
                            int32_t* out_indices, void* out_values, void* workspace,
                            size_t workspace_bytes_, void* stream, int32_t order,
                            bool use_scratch = false) {
    int st = check_rows(logits, dtype, num_rows, width, row_stride, top_k);
    if (st != VTS_OK) return st;
    if (next_n < 1 || compress_ratio < 1 || num_rows % next_n != 0) return VTS_ERR_INVALID;
    if (num_rows == 0) return VTS_OK;
    if (seq_lens == nullptr) return VTS_ERR_INVALID;
    if (out_indices == nullptr || !aligned(out_indices, 16)) return VTS_ERR_INVALID;
    if (out_values && !aligned(out_values, 16)) return VTS_ERR_INVALID;
    const size_t nk = (size_t)num_rows * (size_t)top_k;
    if (out_values && overlap(out_indices, nk * 4, out_values, nk * itemsize(dtype)))
        return VTS_ERR_INVALID;
    int warn = VTS_OK;
    if (pre_idx && !aligned(pre_idx, 16)) {
        pre_idx = nullptr;
        warn = VTS_WARN_HINT_DISCARDED;
    }
    if (order != ORDER_ANY && top_k > NARROW_K_MAX) return VTS_ERR_UNSUPPORTED;
    int32_t slots = slots_for_k(top_k);
    if (use_scratch) {
        slots = scratch_slots(num_rows, width, top_k, dtype);
        if (slots == 0) return VTS_ERR_TOO_LARGE;
    } else {
        st = check_workspace(workspace, workspace_bytes_, num_rows, width, top_k, dtype);
        if (st != VTS_OK) return st;
    }
    int dev = 0, cus = 0;
    st = check_device(stream, &dev, &cus);
    if (st != VTS_OK) return st;
    if (use_scratch) {
        st = scratch_of(dev, &workspace);
        if (st != VTS_OK) return st;
        // the scratch keeps the last call's contents, which may have another
        // layout: clear the counters and row tickets, which must start at zero
        const WsLayout L = ws_layout(num_rows, plan_nsplit(num_rows, width, dtype), slots);
        if (launch_zero(static_cast<uint32_t*>(workspace), L.count / 4,
                        static_cast<hipStream_t>(stream)) != hipSuccess)
            return VTS_ERR_HIP;
    }

    Params p;
    memset(&p, 0, sizeof(p));
    p.x = logits;
    p.row_stride = row_stride;
    p.width = width;
    p.num_rows = (int32_t)num_rows;
    p.k = top_k;
    p.seq_lens = seq_lens;
    p.next_n = next_n;
    p.cr = compress_ratio;
    p.pre_idx = pre_idx;
    p.hint_rung = g_tune.hint_rung;
    p.out_idx = out_indices;
    p.out_vals = out_values;
    p.order = order;
    fill_plan(p, num_rows, width, workspace, slots, dtype, cus);
    log_plan(use_scratch ? "vts_topk_varlen_noalloc"
             : order != ORDER_ANY ? "vts_topk_varlen_ordered" : "vts_topk_varlen",
             p, dtype, width, cus);
    if (launch_varlen(dtype, p, static_cast<hipStream_t>(stream)) != hipSuccess) return VTS_ERR_HIP;
    return warn;
}

int vts_topk_varlen(const void* logits, int32_t dtype, int64_t num_rows, int64_t width,
                    int64_t row_stride, const int32_t* seq_lens, int32_t top_k, int32_t next_n,
                    int32_t compress_ratio, const int32_t* pre_idx, int32_t* out_indices,
                    void* out_values, void* workspace, size_t workspace_bytes_, void* stream) {
    return topk_varlen_impl(logits, dtype, num_rows, width, row_stride, seq_lens, top_k, next_n,
                            compress_ratio, pre_idx, out_indices, out_values, workspace,
                            workspace_bytes_, stream, ORDER_ANY);
}

int vts_topk_varlen_noalloc(const void* logits, int32_t dtype, int64_t num_rows, int64_t width,
                            int64_t row_stride, const int32_t* seq_lens, int32_t top_k,
                            int32_t next_n, int32_t compress_ratio, const int32_t* pre_idx,
                            int32_t* out_indices, void* out_values, void* stream) {
    return topk_varlen_impl(logits, dtype, num_rows, width, row_stride, seq_lens, top_k, next_n,
                            compress_ratio, pre_idx, out_indices, out_values, nullptr, 0,
                            stream, ORDER_ANY, true);
}

int vts_topk_varlen_ordered(const void* logits, int32_t dtype, int64_t num_rows, int64_t width,
                            int64_t row_stride, const int32_t* seq_lens, int32_t top_k,
                            int32_t next_n, int32_t compress_ratio, const int32_t* pre_idx,
                            int32_t* out_indices, void* out_values, void* workspace,
                            size_t workspace_bytes_, void* stream, int32_t tie_break) {
    int32_t order;
    if (!order_of(tie_break, &order)) return VTS_ERR_INVALID;
    return topk_varlen_impl(logits, dtype, num_rows, width, row_stride, seq_lens, top_k, next_n,
                            compress_ratio, pre_idx, out_indices, out_values, workspace,
                            workspace_bytes_, stream, order);
}

static int page_transform_impl(const void* scores, int32_t dtype, int64_t num_rows,
                               int64_t width, int64_t row_stride, const int32_t* lengths,
                               const int32_t* row_starts, const int32_t* src_page_table,
                               int64_t page_table_stride, int64_t page_table_width,
                               const int32_t* page_table_row_starts, int32_t page_size,
                               int32_t top_k, int32_t* out, int32_t* out_raw_indices,
                               void* workspace, size_t workspace_bytes_, void* stream,
                               int32_t order) {
    int st = check_rows(scores, dtype, num_rows, width, row_stride, top_k);
    if (st != VTS_OK) return st;
    if (page_size < 1 || page_size > (1 << 30)) return VTS_ERR_INVALID;
    if (page_table_width < 1 || page_table_stride < page_table_width) return VTS_ERR_INVALID;
    // FlashInfer page-size PR body: with page_size > 1 and row_starts given the
    // page-table starts must be explicit.
    if (page_size > 1 && row_starts && !page_table_row_starts) return VTS_ERR_INVALID;
    if (num_rows == 0) return VTS_OK;
    if (lengths == nullptr || src_page_table == nullptr) return VTS_ERR_INVALID;
    if (out == nullptr || !aligned(out, 16)) return VTS_ERR_INVALID;
    if (out_raw_indices && !aligned(out_raw_indices, 16)) return VTS_ERR_INVALID;
    const size_t nk = (size_t)num_rows * (size_t)top_k;
    if (out_raw_indices && overlap(out, nk * 4, out_raw_indices, nk * 4)) return VTS_ERR_INVALID;
    if (order != ORDER_ANY && top_k > NARROW_K_MAX) return VTS_ERR_UNSUPPORTED;
    st = check_workspace(workspace, workspace_bytes_, num_rows, width, top_k, dtype);
    if (st != VTS_OK) return st;
    int cus = 0;
    st = check_device(stream, nullptr, &cus);
    if (st != VTS_OK) return st;

    Params p;
    memset(&p, 0, sizeof(p));
    p.x = scores;
    p.row_stride = row_stride;
    p.width = width;
    p.num_rows = (int32_t)num_rows;
    p.k = top_k;
    p.next_n = 1;
    p.cr = 1;
    p.lengths = lengths;
    p.row_starts = row_starts;
    p.pt = src_page_table;
    p.pt_stride = page_table_stride;
    p.pt_width = page_table_width;
    p.ptrs = page_table_row_starts;
    p.page_size = page_size;
    p.out_idx = out;
    p.out_raw = out_raw_indices;
    p.order = order;
    fill_plan(p, num_rows, width, workspace, slots_for_k(top_k), dtype, cus);
    log_plan(p.order != ORDER_ANY ? "vts_topk_page_table_transform_ordered" : "vts_topk_page_table_transform", p, dtype, width, cus);
    if (launch_transform(dtype, p, static_cast<hipStream_t>(stream)) != hipSuccess)
        return VTS_ERR_HIP;
    return VTS_OK;
}

int topk_varlen(const void* logits, int32_t dtype, int64_t num_rows, int64_t width,
                int64_t row_stride, const int32_t* seq_lens, int32_t top_k, int32_t next_n,
                int32_t compress_ratio, const int32_t* pre_idx, int32_t* out_indices,
                void* out_values, void* workspace, size_t workspace_bytes_, void* stream) {
    return vts_topk_varlen(logits, dtype, num_rows, width, row_stride, seq_lens, top_k, next_n,
                           compress_ratio, pre_idx, out_indices, out_values, workspace,
                           workspace_bytes_, stream);
}

int topk_page_table_transform(const void* scores, int32_t dtype, int64_t num_rows, int64_t width,
                              int64_t row_stride, const int32_t* lengths,
                              const int32_t* row_starts, const int32_t* src_page_table,
                              int64_t page_table_stride, int64_t page_table_width,
                              const int32_t* page_table_row_starts, int32_t page_size,
                              int32_t top_k, int32_t* out, int32_t* out_raw_indices,
                              void* workspace, size_t workspace_bytes_, void* stream) {
    return vts_topk_page_table_transform(scores, dtype, num_rows, width, row_stride, lengths,
                                         row_starts, src_page_table, page_table_stride,
                                         page_table_width, page_table_row_starts, page_size, top_k,
                                         out, out_raw_indices, workspace, workspace_bytes_, stream);
}

static int ragged_impl(const void* scores, int32_t dtype, int64_t num_rows, int64_t width,
                       int64_t row_stride, const int32_t* lengths, const int32_t* row_starts,
                       const int32_t* topk_indices_offset, int32_t top_k, int32_t* out,
                       int32_t* out_raw_indices, void* workspace, size_t workspace_bytes_,
                       void* stream, int32_t order) {
    int st = check_rows(scores, dtype, num_rows, width, row_stride, top_k);
    if (st != VTS_OK) return st;
    if (num_rows == 0) return VTS_OK;
    if (lengths == nullptr || topk_indices_offset == nullptr) return VTS_ERR_INVALID;
    if (out == nullptr || !aligned(out, 16)) return VTS_ERR_INVALID;
    if (out_raw_indices && !aligned(out_raw_indices, 16)) return VTS_ERR_INVALID;
    const size_t nk = (size_t)num_rows * (size_t)top_k;
    if (out_raw_indices && overlap(out, nk * 4, out_raw_indices, nk * 4)) return VTS_ERR_INVALID;
    if (order != ORDER_ANY && top_k > NARROW_K_MAX) return VTS_ERR_UNSUPPORTED;
    st = check_workspace(workspace, workspace_bytes_, num_rows, width, top_k, dtype);
    if (st != VTS_OK) return st;
    int cus = 0;
    st = check_device(stream, nullptr, &cus);
    if (st != VTS_OK) return st;

    Params p;
    memset(&p, 0, sizeof(p));
    p.x = scores;
    p.row_stride = row_stride;
    p.width = width;
    p.num_rows = (int32_t)num_rows;
    p.k = top_k;
    p.next_n = 1;
    p.cr = 1;
    p.lengths = lengths;
    p.row_starts = row_starts;
    p.offsets = topk_indices_offset;
    p.page_size = 1;
    p.out_idx = out;
    p.out_raw = out_raw_indices;
    p.order = order;
    fill_plan(p, num_rows, width, workspace, slots_for_k(top_k), dtype, cus);
    log_plan(p.order != ORDER_ANY ? "vts_topk_transform_ragged_ordered" : "vts_topk_transform_ragged", p, dtype, width, cus);
    if (launch_transform(dtype, p, static_cast<hipStream_t>(stream)) != hipSuccess)
        return VTS_ERR_HIP;
    return VTS_OK;
}

static int page1_impl(const void* scores, int32_t dtype, int64_t num_rows, int64_t width,
                      int64_t row_stride, const int32_t* lengths, const int32_t* row_starts,
                      const int32_t* page_table, int64_t page_table_stride,
                      int64_t page_table_width, const int32_t* cu_seqlens_q, int64_t num_batches,
                      int32_t top_k, int32_t* out, int32_t* out_raw_indices, void* workspace,
                      size_t workspace_bytes_, void* stream, int32_t order) {
    int st = check_rows(scores, dtype, num_rows, width, row_stride, top_k);
    if (st != VTS_OK) return st;
    if (num_batches < 0 || num_batches > INT32_MAX - 1) return VTS_ERR_INVALID;
    if (page_table_width < 1 || page_table_stride < page_table_width) return VTS_ERR_INVALID;
    if (num_rows == 0) return VTS_OK;
    if (lengths == nullptr || page_table == nullptr || cu_seqlens_q == nullptr)
        return VTS_ERR_INVALID;
    if (out == nullptr || !aligned(out, 16)) return VTS_ERR_INVALID;
    if (out_raw_indices && !aligned(out_raw_indices, 16)) return VTS_ERR_INVALID;
    const size_t nk = (size_t)num_rows * (size_t)top_k;
    if (out_raw_indices && overlap(out, nk * 4, out_raw_indices, nk * 4)) return VTS_ERR_INVALID;
    if (order != ORDER_ANY && top_k > NARROW_K_MAX) return VTS_ERR_UNSUPPORTED;
    st = check_workspace(workspace, workspace_bytes_, num_rows, width, top_k, dtype);
    if (st != VTS_OK) return st;
    int cus = 0;
    st = check_device(stream, nullptr, &cus);
    if (st != VTS_OK) return st;

    Params p;
    memset(&p, 0, sizeof(p));
    p.x = scores;
    p.row_stride = row_stride;
    p.width = width;
    p.num_rows = (int32_t)num_rows;
    p.k = top_k;
    p.next_n = 1;
    p.cr = 1;
    p.lengths = lengths;
    p.row_starts = row_starts;
    p.pt = page_table;
    p.pt_stride = page_table_stride;
    p.pt_width = page_table_width;
    p.page_size = 1;
    p.out_idx = out;
    p.out_raw = out_raw_indices;
    p.order = order;
    fill_plan(p, num_rows, width, workspace, slots_for_k(top_k), dtype, cus);
    log_plan(p.order != ORDER_ANY ? "vts_topk_transform_page1_ordered" : "vts_topk_transform_page1", p, dtype, width, cus);
    const WsLayout L = ws_layout(num_rows, p.nsplit, p.ws_slots);
    int32_t* row_batch = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + L.batch);
    p.row_batch = row_batch;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (launch_row_batch(cu_seqlens_q, (int32_t)num_batches, (int32_t)num_rows, row_batch, s) !=
        hipSuccess)
        return VTS_ERR_HIP;
    if (launch_transform(dtype, p, s) != hipSuccess) return VTS_ERR_HIP;
    return VTS_OK;
}

int vts_topk_page_table_transform(const void* scores, int32_t dtype, int64_t num_rows,
                                  int64_t width, int64_t row_stride, const int32_t* lengths,
                                  const int32_t* row_starts, const int32_t* src_page_table,
                                  int64_t page_table_stride, int64_t page_table_width,
                                  const int32_t* page_table_row_starts, int32_t page_size,
                                  int32_t top_k, int32_t* out, int32_t* out_raw_indices,
                                  void* workspace, size_t workspace_bytes_, void* stream) {
    return page_transform_impl(scores, dtype, num_rows, width, row_stride, lengths, row_starts,
                               src_page_table, page_table_stride, page_table_width,
                               page_table_row_starts, page_size, top_k, out, out_raw_indices,
                               workspace, workspace_bytes_, stream, ORDER_ANY);
}

int vts_topk_page_table_transform_ordered(
    const void* scores, int32_t dtype, int64_t num_rows, int64_t width, int64_t row_stride,
    const int32_t* lengths, const int32_t* row_starts, const int32_t* src_page_table,
    int64_t page_table_stride, int64_t page_table_width, const int32_t* page_table_row_starts,
    int32_t page_size, int32_t top_k, int32_t* out, int32_t* out_raw_indices, void* workspace,
    size_t workspace_bytes_, void* stream, int32_t tie_break) {
    int32_t order;
    if (!order_of(tie_break, &order)) return VTS_ERR_INVALID;
    return page_transform_impl(scores, dtype, num_rows, width, row_stride, lengths, row_starts,
                               src_page_table, page_table_stride, page_table_width,
                               page_table_row_starts, page_size, top_k, out, out_raw_indices,
                               workspace, workspace_bytes_, stream, order);
}

int vts_topk_transform_ragged(const void* scores, int32_t dtype, int64_t num_rows, int64_t width,
                              int64_t row_stride, const int32_t* lengths,
                              const int32_t* row_starts, const int32_t* topk_indices_offset,
                              int32_t top_k, int32_t* out, int32_t* out_raw_indices,
                              void* workspace, size_t workspace_bytes_, void* stream) {
    return ragged_impl(scores, dtype, num_rows, width, row_stride, lengths, row_starts,
                       topk_indices_offset, top_k, out, out_raw_indices, workspace,
                       workspace_bytes_, stream, ORDER_ANY);
}

int vts_topk_transform_ragged_ordered(const void* scores, int32_t dtype, int64_t num_rows,
                                      int64_t width, int64_t row_stride, const int32_t* lengths,
                                      const int32_t* row_starts,
                                      const int32_t* topk_indices_offset, int32_t top_k,
                                      int32_t* out, int32_t* out_raw_indices, void* workspace,
                                      size_t workspace_bytes_, void* stream, int32_t tie_break) {
    int32_t order;
    if (!order_of(tie_break, &order)) return VTS_ERR_INVALID;
    return ragged_impl(scores, dtype, num_rows, width, row_stride, lengths, row_starts,
                       topk_indices_offset, top_k, out, out_raw_indices, workspace,
                       workspace_bytes_, stream, order);
}

int vts_topk_transform_page1(const void* scores, int32_t dtype, int64_t num_rows, int64_t width,
                             int64_t row_stride, const int32_t* lengths, const int32_t* row_starts,
                             const int32_t* page_table, int64_t page_table_stride,
                             int64_t page_table_width, const int32_t* cu_seqlens_q,
                             int64_t num_batches, int32_t top_k, int32_t* out,
                             int32_t* out_raw_indices, void* workspace, size_t workspace_bytes_,
                             void* stream) {
    return page1_impl(scores, dtype, num_rows, width, row_stride, lengths, row_starts, page_table,
                      page_table_stride, page_table_width, cu_seqlens_q, num_batches, top_k, out,
                      out_raw_indices, workspace, workspace_bytes_, stream, ORDER_ANY);
}

int vts_topk_transform_page1_ordered(const void* scores, int32_t dtype, int64_t num_rows,
                                     int64_t width, int64_t row_stride, const int32_t* lengths,
                                     const int32_t* row_starts, const int32_t* page_table,
                                     int64_t page_table_stride, int64_t page_table_width,
                                     const int32_t* cu_seqlens_q, int64_t num_batches,
                                     int32_t top_k, int32_t* out, int32_t* out_raw_indices,
                                     void* workspace, size_t workspace_bytes_, void* stream,
                                     int32_t tie_break) {
    int32_t order;
    if (!order_of(tie_break, &order)) return VTS_ERR_INVALID;
    return page1_impl(scores, dtype, num_rows, width, row_stride, lengths, row_starts, page_table,
                      page_table_stride, page_table_width, cu_seqlens_q, num_batches, top_k, out,
                      out_raw_indices, workspace, workspace_bytes_, stream, order);
}

#ifdef VTS_PHASE_STAMPS
// Phase-timing build only: launches after this call write 16 stamps per unit
// (row unit u at stamps[16u .. 16u + 15]) into `stamps` (device, or null: off).
void vts_phase_stamps(void* stamps) { g_stamps = static_cast<uint64_t*>(stamps); }
#endif

const char* vts_status_string(int status) {
    switch (status) {
        case VTS_OK: return "ok";
        case VTS_WARN_HINT_DISCARDED: return "pre_idx unusable (misaligned); ran without a hint";
        case VTS_ERR_INVALID: return "invalid argument";
        case VTS_ERR_UNSUPPORTED: return "unsupported request or device";
        case VTS_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case VTS_ERR_HIP: return "HIP runtime error";
        case VTS_ERR_TOO_LARGE:
            return "the call needs more device scratch than vts_topk_varlen_noalloc holds (32 MiB)";
    }
    return "unknown status";
}

int vts_workspace_stats(void* workspace, uint32_t* out, int32_t count, void* stream) {
    if (workspace == nullptr || out == nullptr || count < 1) return VTS_ERR_INVALID;
    if (count > 4) count = 4;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(out, workspace, (size_t)count * 4, hipMemcpyDeviceToHost, s) != hipSuccess)
        return VTS_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return VTS_ERR_HIP;
    if (hipMemsetAsync(workspace, 0, 4 * 4, s) != hipSuccess) return VTS_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return VTS_ERR_HIP;
    return VTS_OK;
}

int vts_set_tuning(int32_t key, int64_t value) {
    switch (key) {
        case VTS_TUNE_NSPLIT:
            if (value < 0 || value > MAX_SPLIT) return VTS_ERR_INVALID;
            g_tune.nsplit = (int32_t)value;
            return VTS_OK;
        case VTS_TUNE_FORCE_PATH:
            if (value < 0 || value > 2) return VTS_ERR_INVALID;
            g_tune.force_path = (int32_t)value;
            return VTS_OK;
        case VTS_TUNE_LDS_SLOTS:
            if (value != 0 && (value < 64 || value > CAP)) return VTS_ERR_INVALID;
            g_tune.lds_slots = (int32_t)value;
            return VTS_OK;
        case VTS_TUNE_SPILL_SLOTS:
            if (value != 0 && (value < 64 || value > HI_SLOTS)) return VTS_ERR_INVALID;
            g_tune.spill_slots = (int32_t)value;
            return VTS_OK;
        case VTS_TUNE_SAMPLE_SIGMA:
            if (value < 0 || value > 1000) return VTS_ERR_INVALID;
            g_tune.sigma_tenths = (int32_t)value;
            return VTS_OK;
        case VTS_TUNE_LIKELY_SIGMA:
            if (value < 0 || value > 1000) return VTS_ERR_INVALID;
            g_tune.likely_tenths = (int32_t)value;
            return VTS_OK;
        case VTS_TUNE_NO_BALANCE:
            if (value < 0 || value > 1) return VTS_ERR_INVALID;
            g_tune.no_balance = (int32_t)value;
            return VTS_OK;
        case VTS_TUNE_HINT_RUNG:
            if (value < 0 || value > 1) return VTS_ERR_INVALID;
            g_tune.hint_rung = (int32_t)value;
            return VTS_OK;
        case VTS_TUNE_MIN_CHUNK:
            if (value != 0 && (value < 256 || value > (1 << 20))) return VTS_ERR_INVALID;
            g_tune.min_chunk = (int32_t)value;
            return VTS_OK;
    }
    return VTS_ERR_INVALID;
}

}  // extern "C"
