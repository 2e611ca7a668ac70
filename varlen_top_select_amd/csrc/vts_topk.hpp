// vts_topk.hpp -- exact variable-length top-k selection for gfx950: the kernel
// template and its parts (instantiated by vts_kernels.hip and
// vts_kernels_ordered.hip).
//
// One kernel serves a whole batch.  Each workgroup owns one (row, chunk) unit:
//
//  1. prologue: the row's valid window [base, base + n) is derived on the
//     device -- from seq_lens, next_n and compress_ratio (FlashInfer
//     top_k_varlen doc, `seq_lens`) or from lengths / row_starts (SGLang
//     TopK_Ops, fast_topk_v2).  n == 0 and n <= k rows are answered directly
//     (TensorRT-LLM PR #17821, short-row commit: identity then -1).
//  2. thresholds: a fixed sample of the row (128 blocks of 64 contiguous
//     columns, each on a cache line, or the whole row when it is short) is
//     radix-selected in LDS at two ranks -- a ladder of two rungs, after the
//     sample-calibrated thresholds of the self-sampling GVR V2 description on
//     the TensorRT-LLM PR #17821 page.  The safe rung T is placed so that,
//     for exchangeable data, at least k row elements clear it except with
//     negligible probability; the likely rung T2 >= T so that they clear it
//     in most rows.  All workgroups of a row compute the same rungs.
//  3. filter: one coalesced pass over the unit's columns with 16-byte loads;
//     every key >= T is appended to one candidate list (LDS, then the unit's
//     workspace region) with one wave-aggregated ticket per drained round of
//     staged vectors, and the keys >= T2 are counted.  If the list outgrows
//     its slots, the unit is re-filtered with a compaction filter that keeps
//     at most k candidates at any time (exact for any input, slower).
//  4. verify: if at least k keys cleared T2, the top k are among them and
//     only those are ranked; else, if at least k cleared T, the whole list is
//     ranked; else the row is re-selected over all its columns with the
//     compaction filter (never for exchangeable data: exactness rests on
//     these counts, never on the sample).
//  5. select: the k-th largest candidate key K and the count g of keys > K,
//     by radix select in LDS (10-bit digits from the first differing bit).
//  6. epilogue: all keys > K and k - g keys == K are written (ties are
//     interchangeable); indices are window-relative.  The page-table policy
//     applies the compact transform of the FlashInfer page-size PR body.
//
// Rows long enough get several workgroups (a split row).  Each writes its
// candidates to the workspace, then takes a ticket; the last one merges the
// candidates (steps 4-6) and resets the ticket, leaving the workspace clean.
// No workgroup ever waits for another.

#pragma once

#include <type_traits>

#include "vts_device.hpp"
#include "vts_internal.h"

// Phase stamps, compiled in only for the phase-timing build (-DVTS_PHASE_STAMPS,
// varlen_top_select_amd/phases.py): thread 0 of a workgroup writes the 100 MHz
// real-time counter when the unit starts (0), knows its window (1), has its
// rungs (2), has streamed (3), has written its outputs (4) and has taken its
// split-row ticket (5); slot 6 holds the hardware id (HW_ID | XCC_ID << 32)
// and slot 7 the row and its valid length; the final selection stamps its
// start (8) and the moment its k-th key is known (9); a split row's unit
// stamps the start of its publication (11) and the barrier after it (12),
// and its merging unit the moment it has read the lists' counts (10); the
// emission stamps its output tickets (13) and, with a page table, the staged
// table (14); the sample stamps its arrival (15).
#ifdef VTS_PHASE_STAMPS
#define VTS_STAMP(i)                                                           \
    do {                                                                       \
        if (threadIdx.x == 0 && p.stamps)                                      \
            gstore(p.stamps + (size_t)sm.stamp_unit * VTS_STAMPS_PER_UNIT + (i), \
                   (uint64_t)__builtin_amdgcn_s_memrealtime());                \
    } while (0)
#define VTS_STAMP_ID(row, len)                                                 \
    do {                                                                       \
        if (threadIdx.x == 0 && p.stamps) {                                    \
            gstore(p.stamps + (size_t)sm.stamp_unit * VTS_STAMPS_PER_UNIT + 6, \
                   (uint64_t)__builtin_amdgcn_s_getreg(0xF804) |               \
                       ((uint64_t)__builtin_amdgcn_s_getreg(0xF814) << 32));   \
            gstore(p.stamps + (size_t)sm.stamp_unit * VTS_STAMPS_PER_UNIT + 7, \
                   (uint64_t)(uint32_t)(row) | ((uint64_t)(len) << 32));       \
        }                                                                      \
    } while (0)
#else
#define VTS_STAMP(i) \
    do {             \
    } while (0)
#define VTS_STAMP_ID(row, len) \
    do {                       \
    } while (0)
#endif

namespace vts {

// ---------------------------------------------------------------------------
// row windows and output policies
// ---------------------------------------------------------------------------

// A row's page-table entries [start, start + np) staged in LDS: table[j]
// holds table column start + j for j in [jlo, jhi), the pages that lie inside
// the table; the page size is 2^sh.
struct StagedTable {
    const uint32_t* table;
    uint32_t jlo, jhi, sh;
};

// The outputs of one row as buffer resources over the row's k slots of each
// output array; an array that was not asked for gets an empty resource,
// whose stores the range check drops.  A slot's stores then need only its
// byte offset: no 64-bit address, no test of the array.
struct OutRow {
    __amdgpu_buffer_rsrc_t a, b;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}

struct VarlenPolicy {
    // the output needs no memory reads of its own
    static constexpr bool GATHERS = false;
    // outputs in any order (OrderedVarlenPolicy: canonical order)
    static constexpr bool ORDERED = false;
    // FlashInfer top_k_varlen doc, `seq_lens`: row t of request i ranks its
    // first max(0, (seq_lens[i] - next_n + t + 1) // compress_ratio) columns,
    // clamped to the width.
    // fetch issues the row's loads, finish computes the window from them
    struct Raw {
        int32_t seq;
    };
    __device__ __forceinline__ static Raw fetch(const Params& p, int r) {
        return Raw{gload(p.seq_lens + r / p.next_n)};
    }
    __device__ __forceinline__ static void finish(const Params& p, int r, Raw f, int64_t& base,
                                                  int64_t& n) {
        const int t = r % p.next_n;
        const int64_t num = (int64_t)f.seq - p.next_n + t + 1;  // <= seq when positive
        const int64_t v = num <= 0 ? 0 : (int64_t)((uint32_t)num / (uint32_t)p.cr);
        n = v < p.width ? v : p.width;
        base = 0;
    }
    __device__ __forceinline__ static void window(const Params& p, int r, int64_t& base, int64_t& n) {
        finish(p, r, fetch(p, r), base, n);
    }
    struct Row {};
    __device__ __forceinline__ static Row row(const Params&, int, int64_t) { return Row{}; }
    template <int DT>
    __device__ __forceinline__ static void emit(const Params& p, int r, int64_t base, uint32_t pos, int32_t col,
                                uint32_t raw) {
        const int64_t o = (int64_t)r * p.k + pos;
        gstore(p.out_idx + o, col);
        if (p.out_vals) {
            using raw_t = typename Traits<DT>::raw_t;
            gstore(static_cast<raw_t*>(p.out_vals) + o, (raw_t)raw);
        }
    }
    // row r's outputs: a = indices, b = values
    template <int DT>
    __device__ __forceinline__ static OutRow out_row(const Params& p, int r) {
        using raw_t = typename Traits<DT>::raw_t;
        const int64_t o = (int64_t)r * p.k;
        const uint32_t k = (uint32_t)p.k;
        return OutRow{out_rsrc(p.out_idx + o, k * 4u),
                      p.out_vals ? out_rsrc(static_cast<raw_t*>(p.out_vals) + o, k * (uint32_t)sizeof(raw_t))
                                 : out_rsrc(p.out_idx, 0u)};
    }
    template <int DT>
    __device__ __forceinline__ static void put(const OutRow& o, uint32_t pos, int32_t col, uint32_t raw) {
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)col, o.a, (int)(pos * 4u), 0, 0);
        if constexpr (Traits<DT>::BITS == 32)
            __builtin_amdgcn_raw_buffer_store_b32(raw, o.b, (int)(pos * 4u), 0, 0);
        else
            __builtin_amdgcn_raw_buffer_store_b16((unsigned short)raw, o.b, (int)(pos * 2u), 0, 0);
    }
};

// The deterministic mode of the varlen selection: its own kernels, so the
// sort and the tie-break select add no code to the unordered ones.
struct OrderedVarlenPolicy : VarlenPolicy {
    static constexpr bool ORDERED = true;
};

struct PagePolicy {
    // each output index is read from a table (or an offset) in memory
    static constexpr bool GATHERS = true;
    static constexpr bool ORDERED = false;
    // Window [row_start, row_start + n), n = clamp(length, 0, width - row_start);
    // a start outside [0, width] is an empty row.
    struct Raw {
        int32_t start, len;
    };
    __device__ __forceinline__ static Raw fetch(const Params& p, int r) {
        return Raw{p.row_starts ? gload(p.row_starts + r) : 0, gload(p.lengths + r)};
    }
    __device__ __forceinline__ static void window(const Params& p, int r, int64_t& base, int64_t& n) {
        finish(p, r, fetch(p, r), base, n);
    }
    __device__ __forceinline__ static void finish(const Params& p, int, Raw f, int64_t& base,
                                                  int64_t& n) {
        const int64_t b = f.start;
        const int64_t len = f.len;
        if (b < 0 || b > p.width) {
            base = 0;
            n = 0;
            return;
        }
        const int64_t room = p.width - b;
        base = b;
        n = len < 0 ? 0 : (len > room ? room : len);
    }
    // FlashInfer page-size PR body: out = table[b, start + idx / page_size] *
    // page_size + idx % page_size; -1 stays -1; a table column outside the
    // table also gives -1.
    // The row's own translation inputs, read once per row: a store between
    // two reads of them would make the second wait for it.
    struct Row {
        int64_t start;  // table column of the window's first page
        int32_t add;    // ragged offset
        int32_t b;      // request of the row (page size 1)
    };
    __device__ __forceinline__ static Row row(const Params& p, int r, int64_t base) {
        Row w{base, 0, -1};
        if (p.offsets)
            w.add = gload(p.offsets + r);
        else if (p.row_batch)
            w.b = gload(p.row_batch + r);
        else if (p.ptrs)
            w.start = gload(p.ptrs + r);
        return w;
    }
    // whether translate reads memory (the ragged offset is arithmetic only)
    __device__ __forceinline__ static bool gathers(const Params& p) { return p.offsets == nullptr; }
    __device__ __forceinline__ static int32_t translate(const Params& p, int r, const Row& w, int32_t col) {
        if (col < 0) return -1;
        // SGLang TopK_Ops, fast_topk_transform_ragged_fused: the index plus the
        // row's offset in the ragged KV (int32 arithmetic: caller's contract)
        if (p.offsets) return (int32_t)((uint32_t)col + (uint32_t)w.add);
        // SGLang TopK_Ops, fast_topk_transform_fused: page size 1, the table
        // row of the row's request, the index itself as the table column
        if (p.row_batch) {
            if (w.b < 0 || (int64_t)col >= p.pt_width) return -1;
            return gload(p.pt + (int64_t)w.b * p.pt_stride + col);
        }
        const int64_t pc = w.start + col / p.page_size;
        if (pc < 0 || pc >= p.pt_width) return -1;
        const int64_t page = gload(p.pt + (int64_t)r * p.pt_stride + pc);
        return (int32_t)(page * p.page_size + col % p.page_size);
    }
    // Pages of a window of n columns under a table whose page size P is a
    // power of two (0 where the translation reads no such table): window
    // column c maps to table column start + c / P.
    __device__ __forceinline__ static uint32_t table_pages(const Params& p, int64_t n) {
        if (p.offsets || p.row_batch || (p.page_size & (p.page_size - 1)) != 0) return 0;
        return (uint32_t)((n + p.page_size - 1) / p.page_size);
    }
    __device__ __forceinline__ static StagedTable staged(const Params& p, const Row& w, const uint32_t* table,
                                                    uint32_t np) {
        const int64_t lo = w.start < 0 ? -w.start : 0;
        const int64_t hi = p.pt_width - w.start;
        StagedTable t;
        t.table = table;
        t.jlo = (uint32_t)(lo < (int64_t)np ? lo : (int64_t)np);
        t.jhi = (uint32_t)(hi < (int64_t)t.jlo ? (int64_t)t.jlo : (hi < (int64_t)np ? hi : (int64_t)np));
        t.sh = (uint32_t)__builtin_ctz((uint32_t)p.page_size);
        return t;
    }
    // Issues this thread's loads of the staged entries j = u * NT + thread.
    template <int TJ>
    __device__ __forceinline__ static void table_fetch(const Params& p, int r, const Row& w, const StagedTable& t,
                                                       uint32_t (&tl)[TJ]) {
#pragma unroll
        for (int u = 0; u < TJ; ++u) {
            const uint32_t j = (uint32_t)u * NT + threadIdx.x;
            tl[u] = 0u;
            if (j >= t.jlo && j < t.jhi) tl[u] = (uint32_t)gload(p.pt + (int64_t)r * p.pt_stride + w.start + j);
        }
    }
    // translate from the staged entries (the same bits: the low 32 bits of
    // page * P + col % P), for any 32-bit column and without a branch: a
    // column outside the staged range reads entry 0 (always staged) and
    // yields -1
    __device__ __forceinline__ static int32_t translate_staged(const StagedTable& t, uint32_t col) {
        const uint32_t j = col >> t.sh;
        const bool in = (int32_t)col >= 0 && j >= t.jlo && j < t.jhi;
        const uint32_t e = t.table[in ? j : 0u];
        return in ? (int32_t)((e << t.sh) + (col & ((1u << t.sh) - 1u))) : -1;
    }
    // output slot pos: the raw index col, and the translated index t
    __device__ __forceinline__ static void put_raw(const Params& p, int r, uint32_t pos, int32_t col) {
        if (p.out_raw) gstore(p.out_raw + (int64_t)r * p.k + pos, col);
    }
    __device__ __forceinline__ static void put_idx(const Params& p, int r, uint32_t pos, int32_t t) {
        gstore(p.out_idx + (int64_t)r * p.k + pos, t);
    }
    // row r's outputs: a = translated indices, b = raw indices
    template <int DT>
    __device__ __forceinline__ static OutRow out_row(const Params& p, int r) {
        const int64_t o = (int64_t)r * p.k;
        const uint32_t k = (uint32_t)p.k;
        return OutRow{out_rsrc(p.out_idx + o, k * 4u),
                      p.out_raw ? out_rsrc(p.out_raw + o, k * 4u) : out_rsrc(p.out_idx, 0u)};
    }
    __device__ __forceinline__ static void put_raw(const OutRow& o, uint32_t pos, int32_t col) {
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)col, o.b, (int)(pos * 4u), 0, 0);
    }
    __device__ __forceinline__ static void put_idx(const OutRow& o, uint32_t pos, int32_t t) {
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)t, o.a, (int)(pos * 4u), 0, 0);
    }
};

// The deterministic mode of the windowed selections (kernels of their own).
struct OrderedPagePolicy : PagePolicy {
    static constexpr bool ORDERED = true;
};

// ---------------------------------------------------------------------------
// slices: a unit's columns as scalar head, 16-byte vector body, scalar tail
// ---------------------------------------------------------------------------

struct Slice {
    int64_t h;         // window columns before the first 16-byte boundary
    int64_t v0, v1;    // body vectors [v0, v1), vector v covers columns h + v*VE ...
    int64_t s0, s1;    // scalar columns handled by this unit: [s0, s1) of the head
    int64_t t0, t1;    // and [t0, t1) of the tail
};

template <int DT>
__device__ __forceinline__ Slice make_slice(const typename Traits<DT>::raw_t* row, int64_t n,
                                            int c, int eff) {
    constexpr int VE = Traits<DT>::VE;
    using raw_t = typename Traits<DT>::raw_t;
    Slice s;
    const int64_t mis = (int64_t)(((uintptr_t)row / sizeof(raw_t)) % VE);
    int64_t h = (VE - mis) % VE;
    if (h > n) h = n;
    const int64_t nv = (n - h) / VE;
    s.h = h;
    s.v0 = nv * c / eff;
    s.v1 = nv * (c + 1) / eff;
    s.s0 = 0;
    s.s1 = c == 0 ? h : 0;
    s.t0 = h + nv * VE;
    s.t1 = c == eff - 1 ? n : s.t0;
    return s;
}

// One streaming step: each thread loads U 16-byte vectors, NT vectors apart.
// `vb` points at the unit's first body vector; vector indices are relative to
// it (a unit spans at most 2^31 vectors).
// A unit's body vectors are read through a buffer resource: base in scalar
// registers, a per-thread constant offset plus a wave-uniform step offset, and
// the hardware range check returns zeros past the end (nvec * 16 bytes).  So
// every load of a step is issued unconditionally, with no address arithmetic
// per vector, and the code stays straight-line, which lets the compiler's
// wait counts keep one step's loads in flight while the previous step is
// filtered.  (Rows are below 2^31 bytes, so 32-bit offsets suffice.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t body_rsrc(const void* base, uint32_t bytes) {
    // word 3: the raw-buffer format used for untyped loads on gfx9 parts
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Cache policy of the stream's loads: the non-temporal hint (gfx950
// cache-policy bit NT).  Every byte of the stream is read once, and with the
// hint a plain 16-byte streaming read of 820 MB measured 6.82-6.93 TB/s on
// MI355X against 6.01-6.13 without it (sc0 or sc1 alone: no gain).  The
// sample, whose blocks the stream reads again later, and the workspace lists,
// which the merge and the wide selections read more than once, keep the
// default policy.  (Measured on the 1024 x 262144 fp32 batch, one box: with
// the hint on the sample as well, 143.7-145.1 us warm and 146.7-147.5 cold;
// with the sample on the default policy, 142.0-143.7 and 142.0-144.2.)
constexpr int LOAD_NT = 2;
constexpr int LOAD_SAMPLE = 0;

// Loads one streaming step: vector first + u*NT + threadIdx.x into R[u]
// (zeros past the end).
template <int U>
__device__ __forceinline__ void load_step(u32x4 (&R)[U], __amdgpu_buffer_rsrc_t rs,
                                          uint32_t first) {
#pragma unroll
    for (int u = 0; u < U; ++u)
        R[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rs, (int)(threadIdx.x * 16u),
                                             (int)((first + (uint32_t)u * NT) * 16u), LOAD_NT));
}

// element e (0..VE-1) of a 16-byte vector, as raw bits
template <int DT>
__device__ __forceinline__ uint32_t vec_elem(const u32x4& q, int e) {
    if constexpr (Traits<DT>::VE == 4) {
        return q[e];
    } else {
        return (q[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
    }
}

// ---------------------------------------------------------------------------
// the candidate list of one unit: every key >= T (the safe rung), in arrival
// order; slots [0, lds_cap) in LDS, [lds_cap, hi_cap) in the unit's workspace
// region.  The keys >= T2 (the likely rung) are only counted while streaming:
// the selection ranks the list's keys >= T2 when at least k of them exist and
// all of it otherwise, so no second list is kept.  Keeping the streaming loop
// free of global stores matters: on this target loads and stores share one
// wait counter, and a pending store turns the next wait for a load into a wait
// for every access in flight, which empties the prefetch queue.
// ---------------------------------------------------------------------------

struct Buf {
    uint32_t* gkey;
    uint32_t* gidx;
    uint32_t lds_cap, hi_cap;
};

__device__ __forceinline__ void put_hi(Smem& sm, const Buf& B, uint32_t pos, uint32_t key,
                                       uint32_t col) {
    if (pos < B.lds_cap) {
        sm.key[pos] = key;
        sm.idx[pos] = col;
    } else if (pos < B.hi_cap) {
        gstore_at(B.gkey, pos, key);
        gstore_at(B.gidx, pos, col);
    }
}

// ---------------------------------------------------------------------------
// sampled rungs
// ---------------------------------------------------------------------------

struct Rungs {
    uint32_t T;   // safe rung
    uint32_t T2;  // likely rung, T2 >= T
};

// Short rows are read whole and T = T2 is a lower bound of their k-th largest
// key.  Longer rows read SAMPLE_BLOCKS blocks of SAMPLE_BLOCK columns spread
// evenly over [0, n); with mu = k * SAMPLE / n, the expected number of sampled
// keys above the row's k-th largest,
//   T  = the sample's q-th largest key,  q  = ceil(mu + sigma  * sqrt(mu) + 4),
//   T2 = the sample's q2-th largest key, q2 = ceil(mu + sigma2 * sqrt(mu) + 1).
// Keys are resolved to their top 19 bits for fp32 (a lower bound: every key
// sharing the prefix passes, equal keys included) and exactly for 16-bit keys.
// The loads are issued by sample_load; sample_rungs consumes them.
//
// The sample is read in 16-byte vectors on the row's 16-byte grid (the grid
// starts `mis` elements before the row): a block starts at the first grid
// point at or after its nominal column, and a whole row is the SAMPLE / VE
// grid vectors from the one holding column 0, so "short" means n <= SAMPLE -
// mis.  Four vector loads per thread instead of sixteen scalar ones keep the
// address unit free for the streaming loads that follow.
template <int DT>
struct Sample {
    static constexpr int V = SPT / Traits<DT>::VE;  // vectors per thread
    u32x4 v[V];      // raw bits until sample_rungs turns them into keys
    uint32_t vmask;  // bit j: element j % VE of vector j / VE is a sampled key
    bool whole;      // the whole row is sampled
};

template <int DT>
__device__ __forceinline__ void sample_load(const typename Traits<DT>::raw_t* row, int64_t n,
                                            uint32_t salt, Sample<DT>& S) {
    // One straight run of loads for both cases, all in flight at once; a
    // range-checked buffer over the row's grid vectors returns zeros past the
    // last one, and vmask drops the columns outside [0, n).  Block b starts
    // near (b * span + shift) / 64, shift in [0, span) from the salt: the
    // blocks stay evenly spaced over the row, at an offset that differs from
    // row to row (see StepOrder).
    using raw_t = typename Traits<DT>::raw_t;
    constexpr uint32_t VE = Traits<DT>::VE;
    constexpr int V = Sample<DT>::V;
    constexpr uint32_t VPB = SAMPLE_BLOCK / VE;  // vectors per block
    static_assert(SAMPLE_BLOCK % VE == 0 && (NT * V) % VPB == 0, "whole blocks");
    const uint32_t mis = (uint32_t)(((uintptr_t)row & 15u) / sizeof(raw_t));
    const raw_t* grid = row - mis;  // 16-byte aligned
    const bool whole = n <= (int64_t)(SAMPLE - mis);
    // rows are shorter than 2^31 bytes, so the grid fits a 32-bit range
    const uint32_t nv = (uint32_t)(((uint64_t)n + mis + VE - 1) / VE);
    const __amdgpu_buffer_rsrc_t rs = body_rsrc(grid, nv * 16u);
    // A block starts on a 128-byte line (its grid vector index is congruent
    // to lead mod 8), so its 256 bytes are exactly two cache lines; rounding
    // up moves it at most VE - 1 + 7 * VE columns past its nominal column.
    // Block starts lie in [0, span), so every block ends by column n - 1.
    const uint32_t lead = (8u - (uint32_t)(((uintptr_t)grid >> 4) & 7u)) & 7u;
    const uint64_t span = whole ? 0u : (uint64_t)(n - SAMPLE_BLOCK - (VE - 1) - 7 * VE);
    const uint64_t shift = (salt * span) >> 32;
    S.whole = whole;
    S.vmask = 0;
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const uint32_t g = threadIdx.x + (uint32_t)j * NT;  // 0 .. SAMPLE / VE - 1
        const uint64_t b = g / VPB;
        const uint32_t c = (uint32_t)((b * span + shift) / SAMPLE_BLOCKS);
        const uint32_t g0 = (c + mis + VE - 1) / VE;   // first grid vector at or after c
        const uint32_t gl = g0 + ((lead - g0) & 7u);   // ... on a 128-byte line
        const uint32_t gv = whole ? g : gl + g % VPB;
        S.v[j] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(gv * 16u), 0, LOAD_SAMPLE));
#pragma unroll
        for (uint32_t e = 0; e < VE; ++e) {
            const int64_t col = (int64_t)(gv * VE + e) - (int64_t)mis;
            if (!whole || (col >= 0 && col < n)) S.vmask |= 1u << (j * VE + e);
        }
    }
}

// The M largest of a thread's SPT keys, largest first (an insertion network of
// max/min pairs; every key passes through all M places).
template <int M>
__device__ __forceinline__ void top_m(const uint32_t (&key)[SPT], uint32_t (&t)[M]) {
#pragma unroll
    for (int i = 0; i < M; ++i) t[i] = 0u;
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
        uint32_t x = key[j];
#pragma unroll
        for (int i = 0; i < M; ++i) {
            const uint32_t hi = x > t[i] ? x : t[i];
            x = x > t[i] ? t[i] : x;
            t[i] = hi;
        }
    }
}

// `after_keys` runs once the sampled keys are in registers (the sample loads
// have landed) and before the selection: the caller issues its first
// streaming loads there, so that they neither delay the sample's arrival
// nor wait for the selection.
template <int DT, class AfterKeys>
__device__ __forceinline__ Rungs sample_rungs(Smem& sm, const Params& p, int64_t n,
                                              Sample<DT>& S, AfterKeys after_keys) {
    constexpr int BITS = Traits<DT>::BITS;
    constexpr int VE = Traits<DT>::VE;
    uint32_t q = (uint32_t)p.k, q2 = q;
    if (!S.whole) {
        const float mu = (float)p.k * (float)SAMPLE / (float)n;
        const float sq = sqrtf(mu);
        const float qf = ceilf(mu + p.sigma * sq + 4.0f);
        const float q2f = ceilf(mu + p.sigma2 * sq + 1.0f);
        q = qf >= (float)SAMPLE ? (uint32_t)SAMPLE : (uint32_t)qf;
        q2 = q2f >= (float)q ? q : (uint32_t)q2f;
    }
    uint32_t key[SPT];
#pragma unroll
    for (int j = 0; j < SPT; ++j)
        key[j] = to_key<DT>((typename Traits<DT>::raw_t)vec_elem<DT>(S.v[j / VE], j % VE));
    // the keys exist before anything after this point (the clobber also keeps
    // the caller's loads from being hoisted above it)
#pragma unroll
    for (int j = 0; j < SPT; ++j) __asm__ volatile("" ::"v"(key[j]) : "memory");
    after_keys();
    Rungs R;
    // Every sampled key is valid when the row is not read whole (vmask is
    // full).  Then each thread may keep only its M largest keys and rank the
    // rungs among those M * NT: the result is the sample's own order statistic
    // unless one thread holds more than M of the sample's top q keys, and a
    // lower bound of it otherwise -- a lower rung only admits more candidates,
    // so the rungs stay safe -- with M / SPT of the histogram atomics.
    if (!S.whole && q <= (uint32_t)NT) {
        uint32_t t[4];
        top_m<4>(key, t);
        auto visit4 = [&](auto f) {
#pragma unroll
            for (int i = 0; i < 4; ++i) f(t[i]);
        };
        block_select_pair<BITS, BITS == 32 ? 9 : BITS - RBITS>(sm, visit4, q, q2, R.T, R.T2);
        return R;
    }
    if (!S.whole && q <= (uint32_t)(4 * NT)) {
        uint32_t t[8];
        top_m<8>(key, t);
        auto visit8 = [&](auto f) {
#pragma unroll
            for (int i = 0; i < 8; ++i) f(t[i]);
        };
        block_select_pair<BITS, BITS == 32 ? 9 : BITS - RBITS>(sm, visit8, q, q2, R.T, R.T2);
        return R;
    }
    auto visit = [&](auto f) {
#pragma unroll
        for (int j = 0; j < SPT; ++j)
            if ((S.vmask >> j) & 1u) f(key[j]);
    };
    block_select_pair<BITS, BITS == 32 ? 9 : BITS - RBITS>(sm, visit, q, q2, R.T, R.T2);
    return R;
}

// ---------------------------------------------------------------------------
// the hint: the previous step's selection as a sampling anchor
// ---------------------------------------------------------------------------

// Hint rung (FlashInfer top_k_varlen doc, `pre_idx`: the previous step's top-k
// of the request, used only as a sampling anchor; GVR V2 keeps it as an
// anchor of its sampling, exactness never depending on it).  The row's
// current values are read at every hinted column c and at c + 1 (the pages
// disagree on a +1 shift between steps; reading both serves either
// convention): up to 2k reads, each column counted once (one LDS bit per
// column modulo 2^16 -- a collision only drops a read), hints outside the
// window ignored.  Any k reads at distinct columns are k elements of the row,
// so the k-th largest key among them is a lower bound of the row's k-th
// largest: a rung that never lets fewer than k keys through, and that is
// close to the k-th largest when the hint overlaps the current top k.
constexpr int HINT_J = NARROW_K_MAX / NT;       // hint entries per thread (k <= 2048)
constexpr int HINT_MAP0 = SPREAD_COPIES * SPREAD_STRIDE;  // bitmap after the spread copies
constexpr int HINT_MAP_WORDS = 2048;            // 2^16 bits
static_assert(HINT_MAP0 + HINT_MAP_WORDS <= 2 * CAP, "the hint bitmap fits the candidate arrays");

template <int DT>
struct HintReads {
    int32_t col[HINT_J];
    uint32_t key[2 * HINT_J];
};

// Issues the loads of the hinted columns of request i (the caller waits).
__device__ __forceinline__ void hint_cols(const Params& p, int i, int32_t (&col)[HINT_J]) {
    const int32_t* h = p.pre_idx + (int64_t)i * p.k;
#pragma unroll
    for (int j = 0; j < HINT_J; ++j) {
        const int e = j * NT + (int)threadIdx.x;
        col[j] = e < p.k ? gload(h + e) : -1;
    }
}

// Issues the reads of the row at the hinted columns and c + 1.
template <int DT>
__device__ __forceinline__ void hint_reads(const typename Traits<DT>::raw_t* row, int64_t n,
                                           HintReads<DT>& H) {
#pragma unroll
    for (int j = 0; j < HINT_J; ++j) {
        const uint32_t c0 = (uint32_t)H.col[j], c1 = c0 + 1u;
        const bool v0 = c0 < (uint32_t)n, v1 = v0 && c1 < (uint32_t)n;
        H.key[2 * j] = v0 ? to_key<DT>(gload(row + c0)) : 0u;
        H.key[2 * j + 1] = v1 ? to_key<DT>(gload(row + c1)) : 0u;
    }
}

// The hint rung from the reads (every thread calls; leaves the spread copies
// and the bitmap dirty: the caller clears them before the sample select).
template <int DT>
__device__ __forceinline__ uint32_t hint_rung(Smem& sm, const Params& p, int64_t n,
                                              HintReads<DT>& H) {
    constexpr int BITS = Traits<DT>::BITS;
    uint32_t* map = sm.cand_words + HINT_MAP0;
    uint32_t keep = 0;  // bit e: read e is the first read of its column
#pragma unroll
    for (int j = 0; j < HINT_J; ++j) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t c = (uint32_t)H.col[j] + (uint32_t)h;
            if ((uint32_t)H.col[j] < (uint32_t)n && c < (uint32_t)n) {
                const uint32_t b = c & 0xFFFFu, m = 1u << (b & 31u);
                if (!(atomicOr(&map[b >> 5], m) & m)) keep |= 1u << (2 * j + h);
            }
        }
    }
    lds_sync();
    uint32_t t1, t2;
    block_select_pair<BITS, BITS == 32 ? 9 : BITS - RBITS>(
        sm,
        [&](auto f) {
#pragma unroll
            for (int e = 0; e < 2 * HINT_J; ++e) f(((keep >> e) & 1u) ? H.key[e] : 0u);
        },
        (uint32_t)p.k, (uint32_t)p.k, t1, t2);
    return t1;
}

// Zeroes the hint bitmap.
__device__ __forceinline__ void hint_map_clear(Smem& sm) {
    for (int j = threadIdx.x; j < HINT_MAP_WORDS; j += NT) sm.cand_words[HINT_MAP0 + j] = 0;
}

// ---------------------------------------------------------------------------
// fast filter: one pass, no barriers inside the loop
// ---------------------------------------------------------------------------

// key of element e of q when the element is known to be >= +0
template <int DT>
__device__ __forceinline__ uint32_t nonneg_key(const u32x4& q, int e) {
    if constexpr (Traits<DT>::BITS == 32) {
        return q[e] | 0x80000000u;
    } else {
        const uint32_t w = q[e >> 1];
        return ((e & 1) ? (w >> 16) : (w & 0xFFFFu)) | 0x8000u;
    }
}

// Keys of one kernel: order-preserving keys, canonical ones (canon_key) in
// the deterministic mode.
template <int DT, bool CANON>
struct Keys {
    __device__ __forceinline__ static uint32_t of(uint32_t raw) {
        const uint32_t k = to_key<DT>(raw);
        return CANON ? canon_key<DT>(k) : k;
    }
    // element e of q, known to be >= +0 (only a NaN's key can change)
    __device__ __forceinline__ static uint32_t of_nonneg(const u32x4& q, int e) {
        const uint32_t k = nonneg_key<DT>(q, e);
        return CANON ? canon_key<DT>(k) : k;
    }
};

// Rung tests on an element's raw bits.  With FAST (both rungs >= +0, the
// normal case) "key >= T" is a signed compare of the raw bits with the
// rung's raw bits: non-negative values order like their bits and negative
// ones are negative integers.  Otherwise the order-preserving key is formed.
template <int DT, bool FAST, bool CANON>
struct RungTest {
    int32_t a, a2;  // FAST: the rungs' raw bits, sign-extended
    uint32_t t, t2; // otherwise: the rungs as keys
    __device__ __forceinline__ explicit RungTest(const Rungs& G) {
        if constexpr (Traits<DT>::BITS == 32) {
            a = (int32_t)(G.T & 0x7FFFFFFFu);
            a2 = (int32_t)(G.T2 & 0x7FFFFFFFu);
        } else {
            a = (int32_t)(G.T & 0x7FFFu);
            a2 = (int32_t)(G.T2 & 0x7FFFu);
        }
        t = G.T;
        t2 = G.T2;
    }
    // element e of vector q: *in = key >= T, *up = key >= T2
    __device__ __forceinline__ void operator()(const u32x4& q, int e, bool& in, bool& up) const {
        if constexpr (FAST) {
            int32_t v;
            if constexpr (Traits<DT>::BITS == 32) {
                v = (int32_t)q[e];
            } else {
                const uint32_t w = q[e >> 1];
                v = (e & 1) ? ((int32_t)w >> 16) : (int32_t)(int16_t)(w & 0xFFFFu);
            }
            in = v >= a;
            up = v >= a2;
        } else {
            const uint32_t key = Keys<DT, CANON>::of(vec_elem<DT>(q, e));
            in = key >= t;
            up = key >= t2;
        }
    }
};

// Raw bits that fail every raw-bit rung test (a negative integer in both
// halves for 16-bit elements); a partial last step is padded with them.
template <int DT>
__device__ __forceinline__ constexpr uint32_t fail_word() {
    return Traits<DT>::BITS == 32 ? 0x80000000u : 0x80008000u;
}


// Filters one streaming step in two passes over the thread's U vectors.
// Pass 1 counts: each compare yields a 64-lane mask (ballot), so the wave's
// totals are scalar popcounts; one LDS ticket then reserves the wave's slots
// and the keys >= T2 are added to `upc` (the wave's count).  Pass 2 repeats
// the compares and, only for elements whose mask is non-empty, writes each
// candidate at the ticket base plus its rank among the wave's lanes (mbcnt).
// With FAST every vector of the step is valid (a partial step has been padded
// with fail_word).
template <int DT, bool FAST, bool CANON>
__device__ __forceinline__ void filter_step(Smem& sm, const Buf& B,
                                            u32x4 (&R)[Traits<DT>::U], uint32_t first,
                                            uint32_t nvec, uint32_t col0,
                                            const RungTest<DT, FAST, CANON>& test, uint32_t& upc) {
    constexpr int VE = Traits<DT>::VE;
    constexpr int U = Traits<DT>::U;
    uint32_t ti = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool ok = FAST || first + (uint32_t)u * NT + threadIdx.x < nvec;
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            bool in, up;
            test(R[u], e, in, up);
            uint64_t mi = ballot(in), mh = ballot(up);
            if constexpr (!FAST) {
                const uint64_t okm = ballot(ok);
                mi &= okm;
                mh &= okm;
            }
            ti += (uint32_t)__popcll(mi);
            upc += (uint32_t)__popcll(mh);  // T2 >= T: the upper keys are among them
        }
    }
    if (ti == 0) return;  // uniform
    uint32_t bh = 0;
    if (lane_id() == 0) bh = atomicAdd(&sm.cand_n, ti);
    bh = first_lane_value(bh);
    // the compares are redone below rather than kept: holding every mask of
    // the first pass would take more scalar registers than there are
#pragma unroll
    for (int u = 0; u < U; ++u) __asm__ volatile("" : "+v"(R[u]));
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t v = first + (uint32_t)u * NT + threadIdx.x;
        const bool ok = FAST || v < nvec;
        const uint32_t colu = col0 + v * VE;
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            bool in, up;
            test(R[u], e, in, up);
            const bool h = ok && in;
            const uint64_t mi = ballot(h);
            if (mi == 0) continue;  // uniform
            const uint32_t key = FAST ? Keys<DT, CANON>::of_nonneg(R[u], e)
                                      : Keys<DT, CANON>::of(vec_elem<DT>(R[u], e));
            const uint32_t col = colu + (uint32_t)e;
            const uint32_t nh = (uint32_t)__popcll(mi);
            if (bh + nh <= B.lds_cap) {  // uniform: the usual case
                if (h) {
                    const uint32_t pos = bh + mbcnt(mi);
                    sm.key[pos] = key;
                    sm.idx[pos] = col;
                }
            } else if (h) {
                put_hi(sm, B, bh + mbcnt(mi), key, col);
            }
            bh += nh;
        }
    }
}

// Pads the vectors of a partial step that lie past the unit's end.
template <int DT>
__device__ __forceinline__ void pad_step(u32x4 (&R)[Traits<DT>::U], uint32_t first,
                                         uint32_t nvec) {
    constexpr uint32_t F = fail_word<DT>();
#pragma unroll
    for (int u = 0; u < Traits<DT>::U; ++u)
        if (first + (uint32_t)u * NT + threadIdx.x >= nvec) R[u] = u32x4{F, F, F, F};
}

// Largest element of a vector as a signed integer of its raw bits: the
// raw-bit rung test passes for some element exactly when it passes for this.
typedef short s16x2 __attribute__((ext_vector_type(2)));
template <int DT>
__device__ __forceinline__ int32_t vec_max_raw(const u32x4& q) {
    if constexpr (Traits<DT>::BITS == 32) {
        const int32_t a = (int32_t)q[0] > (int32_t)q[1] ? (int32_t)q[0] : (int32_t)q[1];
        const int32_t b = (int32_t)q[2] > (int32_t)q[3] ? (int32_t)q[2] : (int32_t)q[3];
        return a > b ? a : b;
    } else {
        // (each word copied out first: a bit cast of a vector element
        // expression is not reliable with this compiler)
        const uint32_t w0 = q[0], w1 = q[1], w2 = q[2], w3 = q[3];
        const s16x2 m = __builtin_elementwise_max(
            __builtin_elementwise_max(__builtin_bit_cast(s16x2, w0), __builtin_bit_cast(s16x2, w1)),
            __builtin_elementwise_max(__builtin_bit_cast(s16x2, w2), __builtin_bit_cast(s16x2, w3)));
        return m.x > m.y ? (int32_t)m.x : (int32_t)m.y;
    }
}

// Drains the first sc entries of a wave's staging queue (sc <= 64,
// wave-uniform), which start at slot `head` of the wave's ring, in one round:
// lane l takes entry l and runs the element filter on its vector;
// the candidates get one LDS ticket as in filter_step and the keys >= T2 are
// added to `upc`.  Every lane of the wave calls it; no barrier (the queue is
// the wave's own).
template <int DT, bool CANON>
__device__ __forceinline__ void drain_stage(Smem& sm, const Buf& B, uint32_t col0,
                                            const RungTest<DT, true, CANON>& test, uint32_t sc,
                                            uint32_t head, uint32_t& upc) {
    constexpr int VE = Traits<DT>::VE;
    constexpr uint32_t F = fail_word<DT>();
    const uint32_t base = (threadIdx.x >> 6) * STAGE;
    const uint32_t l = lane_id();
    u32x4 q = u32x4{F, F, F, F};
    uint32_t v = 0;
    if (l < sc) {
        const uint32_t slot = base + ((head + l) & (STAGE - 1));
        q = sm.stage.vec[slot];
        v = sm.stage.v[slot];
    }
    uint32_t ti = 0;
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        bool in, up;
        test(q, e, in, up);
        ti += (uint32_t)__popcll(ballot(in));  // > 0: a staged vector holds a candidate
        upc += (uint32_t)__popcll(ballot(up));
    }
    uint32_t bh = 0;
    if (l == 0) bh = atomicAdd(&sm.cand_n, ti);
    bh = first_lane_value(bh);
    const uint32_t colv = col0 + v * VE;
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        bool in, up;
        test(q, e, in, up);
        const uint64_t mi = ballot(in);
        if (mi == 0) continue;  // uniform
        if (in) put_hi(sm, B, bh + mbcnt(mi), Keys<DT, CANON>::of_nonneg(q, e), colv + (uint32_t)e);
        bh += (uint32_t)__popcll(mi);
    }
}

// One streaming step with both rungs >= +0.  Per vector: the largest raw
// element against the safe rung T; the (few) vectors holding a candidate are
// appended to the wave's staging queue in LDS (ballot + mbcnt positions), a
// ring of STAGE slots whose sc entries start at slot `head`.  Whenever
// STAGE_DRAIN are queued, a round of STAGE_DRAIN is drained from the head,
// which then moves on by STAGE_DRAIN (so it is 0 or STAGE_DRAIN), and the
// per-element work runs on rounds of staged vectors instead of on every
// element of the step.
template <int DT, bool CANON>
__device__ __forceinline__ void stage_step(Smem& sm, const Buf& B, const u32x4 (&R)[Traits<DT>::U],
                                           uint32_t first, uint32_t col0,
                                           const RungTest<DT, true, CANON>& test, uint32_t& sc,
                                           uint32_t& head, uint32_t& upc) {
    // Drains run while at least STAGE_DRAIN vectors are queued, so a vector's
    // 64 writes start at sc <= STAGE_DRAIN - 1 entries past the head and end
    // before it comes round again: the queued entries are never overwritten.
    static_assert(STAGE_DRAIN - 1 + 64 <= STAGE && STAGE_DRAIN <= 64, "staging queue bound");
    static_assert(STAGE == 2 * STAGE_DRAIN && (STAGE & (STAGE - 1)) == 0, "ring of two rounds");
    const uint32_t base = (threadIdx.x >> 6) * STAGE;
    const uint32_t l = lane_id();
#pragma unroll
    for (int u = 0; u < Traits<DT>::U; ++u) {
        const bool hit = vec_max_raw<DT>(R[u]) >= test.a;
        const uint64_t m = ballot(hit);
        const uint32_t nh = (uint32_t)__popcll(m);
        // Every lane writes, without branching: hits to entries [sc, sc + nh)
        // in lane order, the others to [sc + nh, sc + 64), which later entries
        // overwrite and the drain never reads.
        const uint32_t below = mbcnt(m);
        const uint32_t pos = base + ((head + sc + (hit ? below : nh + (l - below))) & (STAGE - 1));
        sm.stage.vec[pos] = R[u];
        sm.stage.v[pos] = first + (uint32_t)u * NT + threadIdx.x;
        sc += nh;
        if (sc >= (uint32_t)STAGE_DRAIN) {  // (sc < 2 * STAGE_DRAIN: one round at most)
            drain_stage<DT, CANON>(sm, B, col0, test, STAGE_DRAIN, head, upc);
            sc -= STAGE_DRAIN;
            head ^= (uint32_t)STAGE_DRAIN;
        }
    }
}

// The streaming loop over a unit's body vectors, starting with step 0 already
// in RA (or in flight to it): two register sets in turn, the next step's loads
// are in flight while the current one is filtered.  FAST (both rungs >= +0)
// uses the staged vector filter, otherwise the element filter.
// Order in which a unit visits its steps: step s is the body's step
// (s + rot) mod nsteps.  Units start their streams at spread-out offsets
// (rot from a hash of the unit index), so at any moment the workgroups of a
// batch read different address ranges of their rows instead of all reading
// the same offset of equally spaced rows, which would load a few HBM channels
// and leave the rest idle.
// A step s >= nsteps (the loop's last prefetch) maps past the unit's body,
// where the buffer's range check answers every load with zeros without a
// memory access.
struct StepOrder {
    uint32_t nsteps, rot;
    __device__ __forceinline__ uint32_t first(uint32_t s, uint32_t step) const {
        if (s >= nsteps) return nsteps * step;
        uint32_t t = s + rot;
        if (t >= nsteps) t -= nsteps;
        return t * step;
    }
};

__device__ __forceinline__ uint32_t spread_hash(uint32_t x) { return x * 0x9E3779B1u; }

// The streaming loop over a unit's body vectors, starting with the first step
// of `order` already in RA (or in flight to it): two register sets in turn,
// the next step's loads are in flight while the current one is filtered.
// FAST (both rungs >= +0) uses the staged vector filter, otherwise the element
// filter.
template <int DT, bool FAST, bool CANON>
__device__ __forceinline__ void stream_unit(Smem& sm, const Buf& B, u32x4 (&RA)[Traits<DT>::U],
                                            u32x4 (&RB)[Traits<DT>::U],
                                            __amdgpu_buffer_rsrc_t rs, uint32_t nvec,
                                            uint32_t col0, const Rungs& G, const StepOrder& order) {
    constexpr uint32_t STEP = (uint32_t)NT * Traits<DT>::U;
    const RungTest<DT, FAST, CANON> test(G);
    uint32_t sc = 0;    // staged vectors of this wave (FAST)
    uint32_t head = 0;  // first staged slot of the wave's ring (FAST)
    uint32_t upc = 0;   // keys >= T2 seen by this wave
    auto step = [&](u32x4 (&R)[Traits<DT>::U], uint32_t vs) {
        if constexpr (FAST) {
            if (vs + STEP > nvec) pad_step<DT>(R, vs, nvec);
            stage_step<DT, CANON>(sm, B, R, vs, col0, test, sc, head, upc);
        } else {
            filter_step<DT, false, CANON>(sm, B, R, vs, nvec, col0, test, upc);
        }
    };
    // On entry the loads of the first step (RA) are in flight.  The first step
    // is filtered before the loop, so on entry and on the back edge alike
    // exactly the loads of RB are in flight at the loop header: the compiler's
    // wait counts then let them stay in flight while RA is filtered.  (The
    // loads for the step past the last one fall outside the buffer: zeros,
    // no memory traffic.)
    const uint32_t ns = order.nsteps;
    load_step(RB, rs, order.first(1, STEP));
    step(RA, order.first(0, STEP));
    for (uint32_t s = 1; s < ns; s += 2) {
        load_step(RA, rs, order.first(s + 1, STEP));
        step(RB, order.first(s, STEP));
        if (s + 1 >= ns) break;
        load_step(RB, rs, order.first(s + 2, STEP));
        step(RA, order.first(s + 1, STEP));
    }
    if constexpr (FAST) {
        if (sc) drain_stage<DT, CANON>(sm, B, col0, test, sc, head, upc);
    }
    if (lane_id() == 0 && upc) atomicAdd(&sm.up_n, upc);
}

// scalar columns [a, b) of the window (at most a few), every thread calls
template <int DT, bool CANON>
__device__ __forceinline__ void filter_scalars(Smem& sm, const Buf& B,
                                               const typename Traits<DT>::raw_t* row, int64_t a,
                                               int64_t b, const Rungs& G) {
    for (int64_t base = a; base < b; base += NT) {
        const int64_t c = base + threadIdx.x;
        const bool ok = c < b;
        const uint32_t key = ok ? Keys<DT, CANON>::of(gload(row + c)) : 0u;
        const bool in = ok && key >= G.T;
        const uint64_t mu = ballot(ok && key >= G.T2);
        if (lane_id() == 0 && mu) atomicAdd(&sm.up_n, (uint32_t)__popcll(mu));
        const uint32_t pos = wave_ticket_n(&sm.cand_n, in ? 1u : 0u);
        if (in) put_hi(sm, B, pos, key, (uint32_t)c);
    }
}

// ---------------------------------------------------------------------------
// compaction filter: exact for any input; keeps at most CAP candidates in LDS
// ---------------------------------------------------------------------------

// Entry threshold of the compaction filter.  Unordered: key > T (strict) or
// key >= T.  ORD (deterministic mode): entries are ranked by (key, tie
// column), the tie column being ~col for the SMALL tie-break and col for
// LARGE, so that the larger pair wins; columns are distinct, so this order is
// total and its top k is the unique deterministic selection.  An entry then
// passes when its pair is above (T, C), or equal to it when not strict.
// Initially C = 0 and not strict: key >= T, as unordered.
template <bool ORD>
struct Thr {
    uint32_t T;
    bool strict;
    uint32_t C = 0u;
    bool small = false;
    __device__ __forceinline__ uint32_t tie(uint32_t col) const { return small ? ~col : col; }
    __device__ __forceinline__ bool pass(uint32_t key, uint32_t col) const {
        if constexpr (ORD) {
            if (key != T) return key > T;
            return strict ? tie(col) > C : tie(col) >= C;
        } else {
            return strict ? key > T : key >= T;
        }
    }
};

template <bool ORD>
__device__ __forceinline__ Thr<ORD> make_thr(const Params& p, uint32_t T) {
    Thr<ORD> t{T, false};
    t.small = (p.order & 3) == ORDER_SMALL;
    return t;
}

// Reduces LDS slots [0, cand_n) plus the calling threads' register entries that
// pass `thr` to exactly k entries: the top k of that union -- all keys > K and
// enough keys == K, where K is the k-th largest key (ORD: of the keys == K
// those with the largest tie columns, so the k entries are the top k under the
// total order).  Afterwards only entries above the k-th can matter.
template <int DT, int KPT, bool ORD>
__device__ __forceinline__ void compact(Smem& sm, int k, const uint32_t (&kk)[KPT],
                                        const uint32_t (&cc)[KPT], uint32_t vm, Thr<ORD>& thr,
                                        uint32_t old_n) {
    uint32_t K, gt;
    block_select_exact(
        sm,
        [&](auto f) {
            for (uint32_t q = threadIdx.x; q < old_n; q += NT) f(sm.key[q]);
#pragma unroll
            for (int j = 0; j < KPT; ++j)
                if (((vm >> j) & 1u) && thr.pass(kk[j], cc[j])) f(kk[j]);
        },
        (uint32_t)k, K, gt);
    const uint32_t need_eq = (uint32_t)k - gt;
    // ORD: the need_eq-th largest tie column C among the keys == K; exactly
    // need_eq of them have a tie column >= C
    uint32_t C = 0u;
    if constexpr (ORD) {
        uint32_t cgt;
        block_select_exact(
            sm,
            [&](auto f) {
                for (uint32_t q = threadIdx.x; q < old_n; q += NT)
                    if (sm.key[q] == K) f(thr.tie(sm.idx[q]));
#pragma unroll
                for (int j = 0; j < KPT; ++j)
                    if (((vm >> j) & 1u) && thr.pass(kk[j], cc[j]) && kk[j] == K) f(thr.tie(cc[j]));
            },
            need_eq, C, cgt);
    }
    auto keep_eq = [&](uint32_t col, uint32_t e) {
        if constexpr (ORD) {
            return thr.tie(col) >= C;
        } else {
            return e < need_eq;
        }
    };
    if (threadIdx.x == 0) {
        sm.cnt_a = 0;
        sm.cnt_b = 0;
    }
    __syncthreads();
    // In-place rewrite, one round of NT slots at a time: a kept entry goes to a
    // slot below the number of entries read so far, so no unread slot is hit.
    const uint32_t rounds = (old_n + NT - 1) / NT;
    for (uint32_t rd = 0; rd < rounds; ++rd) {
        const uint32_t q = rd * NT + threadIdx.x;
        const bool ok = q < old_n;
        const uint32_t key = ok ? sm.key[q] : 0u;
        const uint32_t col = ok ? sm.idx[q] : 0u;
        __syncthreads();
        uint64_t m;
        const bool iseq = ok && key == K;
        const uint32_t e = wave_ticket(&sm.cnt_b, iseq, m);
        const bool keep = (ok && key > K) || (iseq && keep_eq(col, e));
        const uint32_t pos = wave_ticket(&sm.cnt_a, keep, m);
        if (keep) {
            sm.key[pos] = key;
            sm.idx[pos] = col;
        }
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const bool ok = ((vm >> j) & 1u) && thr.pass(kk[j], cc[j]);
        uint64_t m;
        const bool iseq = ok && kk[j] == K;
        const uint32_t e = wave_ticket(&sm.cnt_b, iseq, m);
        const bool keep = (ok && kk[j] > K) || (iseq && keep_eq(cc[j], e));
        const uint32_t pos = wave_ticket(&sm.cnt_a, keep, m);
        if (keep) {
            sm.key[pos] = kk[j];
            sm.idx[pos] = cc[j];
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) sm.cand_n = (uint32_t)k;
    __syncthreads();
    thr.T = K;
    thr.C = C;
    thr.strict = true;
}

// One compaction-filter step over register entries kk / cc (valid mask vm).
template <int DT, int KPT, bool ORD>
__device__ __forceinline__ void careful_step(Smem& sm, int k, const uint32_t (&kk)[KPT],
                                             const uint32_t (&cc)[KPT], uint32_t vm,
                                             Thr<ORD>& thr) {
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) cnt += (((vm >> j) & 1u) && thr.pass(kk[j], cc[j])) ? 1u : 0u;
    uint32_t cand;
    const uint32_t total = block_sum(sm, cnt, cand);
    if (total == 0) return;
    if (cand + total > (uint32_t)CAP) {
        compact<DT, KPT, ORD>(sm, k, kk, cc, vm, thr, cand);
        return;
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const bool ok = ((vm >> j) & 1u) && thr.pass(kk[j], cc[j]);
        uint64_t m;
        const uint32_t pos = wave_ticket(&sm.cand_n, ok, m);
        if (ok) {
            sm.key[pos] = kk[j];
            sm.idx[pos] = cc[j];
        }
    }
    __syncthreads();
}

// Compaction filter over a whole slice; leaves the candidates in LDS slots
// [0, sm.cand_n), sm.cand_n <= CAP, containing every key > the final threshold
// and, if the slice has at least k keys passing thr0, a top-k of the slice.
template <int DT, bool ORD>
__device__ __forceinline__ void careful_filter(Smem& sm, const Params& p, const typename Traits<DT>::raw_t* row,
                               const Slice& s, Thr<ORD> thr) {
    constexpr int VE = Traits<DT>::VE;
    if (threadIdx.x == 0) sm.cand_n = 0;
    __syncthreads();
    // scalar head and tail columns, as one step each
    for (int part = 0; part < 2; ++part) {
        const int64_t a = part == 0 ? s.s0 : s.t0;
        const int64_t b = part == 0 ? s.s1 : s.t1;
        for (int64_t base = a; base < b; base += NT) {
            uint32_t kk[1], cc[1];
            const int64_t c = base + threadIdx.x;
            const uint32_t vm = c < b ? 1u : 0u;
            kk[0] = vm ? Keys<DT, ORD>::of(gload(row + c)) : 0u;
            cc[0] = (uint32_t)c;
            careful_step<DT, 1, ORD>(sm, p.k, kk, cc, vm, thr);
        }
    }
    // one 16-byte vector per thread per step: this path is rare, keep it lean
    const u32x4* vb = reinterpret_cast<const u32x4*>(row + s.h);
    for (int64_t vs = s.v0; vs < s.v1; vs += NT) {
        const int64_t v = vs + threadIdx.x;
        u32x4 q = {0u, 0u, 0u, 0u};
        if (v < s.v1) q = gload(vb + v);
        uint32_t kk[VE], cc[VE];
        const uint32_t vm = v < s.v1 ? ((1u << VE) - 1u) : 0u;
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            kk[e] = Keys<DT, ORD>::of(vec_elem<DT>(q, e));
            cc[e] = (uint32_t)(s.h + v * VE + e);
        }
        careful_step<DT, VE, ORD>(sm, p.k, kk, cc, vm, thr);
    }
}

// Adds the workspace entries gk[0, m) / gi[0, m) (all passing thr) to the LDS
// candidates [0, sm.cand_n) with the compaction filter, E entries per thread per
// round: all loads of a round are issued before any is used.
template <int DT, bool ORD>
__device__ __forceinline__ void ingest_global(Smem& sm, int k, const uint32_t* gk,
                                              const uint32_t* gi, uint32_t m, Thr<ORD>& thr) {
    constexpr int E = 8;
    for (uint32_t b = 0; b < m; b += (uint32_t)NT * E) {
        uint32_t kk[E], cc[E], vm = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint32_t q = b + (uint32_t)e * NT + threadIdx.x;
            const uint32_t qc = q < m ? q : m - 1;
            kk[e] = gload(gk + qc);
            cc[e] = gload(gi + qc);
            if (q < m) vm |= 1u << e;
        }
        careful_step<DT, E, ORD>(sm, k, kk, cc, vm, thr);
    }
}

// ---------------------------------------------------------------------------
// final selection and epilogue
// ---------------------------------------------------------------------------

// registers per thread that hold every on-chip candidate slot
constexpr int ONCHIP_J = (CAP + NT - 1) / NT;

// Enumerates candidate entries (key, col) with wave-uniform trip counts.
// The first `own` entries come from LDS slots [0, own), the rest, up to n,
// from slots [own, n) of a workspace list (a unit's spilled candidates); all
// are read once into registers (entry j * NT + threadIdx.x in register j), so
// the selection passes and the emission visit registers.  Only keys >= thr
// are visited.  n <= J * NT: J = 15 covers the on-chip slots, the default
// J = 20 a list with up to 5120 entries.
template <int J = 20>
struct LdsSrc {
    static_assert(J * NT >= CAP, "every on-chip slot has a register");
    uint32_t n, thr;
    uint32_t key[J], idx[J];
    __device__ __forceinline__ LdsSrc(Smem& sm, uint32_t n_, uint32_t thr_ = 0u)
        : n(n_), thr(thr_) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const uint32_t q = (uint32_t)j * NT + threadIdx.x;
            key[j] = q < n ? sm.key[q] : 0u;
            idx[j] = q < n ? sm.idx[q] : 0u;
        }
    }
    __device__ __forceinline__ LdsSrc(Smem& sm, uint32_t own, const uint32_t* gkey,
                                      const uint32_t* gidx, uint32_t n_, uint32_t thr_)
        : n(n_), thr(thr_) {
        // every load of both parts is issued before any is used; only the
        // spilled slots [own, n) are read from the workspace
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const uint32_t q = (uint32_t)j * NT + threadIdx.x;
            key[j] = 0u;
            idx[j] = 0u;
            if (q < own) {
                key[j] = sm.key[q];
                idx[j] = sm.idx[q];
            } else if (q < n) {
                key[j] = gload(gkey + q);
                idx[j] = gload(gidx + q);
            }
        }
    }
    static constexpr int SLOTS = J;
    template <class F>
    __device__ __forceinline__ void for_each(Smem&, F f) const {
#pragma unroll
        for (int j = 0; j < J; ++j)
            f((uint32_t)j * NT + threadIdx.x < n && key[j] >= thr, key[j], idx[j]);
    }
    // the same, with the register index j as the first argument
    template <class F>
    __device__ __forceinline__ void for_each_slot(F f) const {
#pragma unroll
        for (int j = 0; j < J; ++j)
            f(j, (uint32_t)j * NT + threadIdx.x < n && key[j] >= thr, key[j], idx[j]);
    }
};

// ---------------------------------------------------------------------------
// wide selections (top_k > 2048): candidate lists too long for the registers
// are enumerated from LDS and the workspace on every visit
// ---------------------------------------------------------------------------

constexpr int WIDE_B = 16;  // workspace entries per thread in flight per round

// Visits workspace entries gk[from, n) / gi[from, n), WIDE_B per thread per
// round with all loads of a round issued before any is used (the entries are
// in L2: a unit wrote them during its stream).
template <class F>
__device__ __forceinline__ void visit_global(const uint32_t* gk, const uint32_t* gi, uint32_t from,
                                             uint32_t n, F f) {
    for (uint32_t q0 = from; q0 < n; q0 += (uint32_t)NT * WIDE_B) {
        uint32_t kk[WIDE_B], cc[WIDE_B];
#pragma unroll
        for (int b = 0; b < WIDE_B; ++b) {
            const uint32_t q = q0 + (uint32_t)b * NT + threadIdx.x;
            const uint32_t qc = q < n ? q : from;
            kk[b] = gload(gk + qc);
            cc[b] = gload(gi + qc);
        }
#pragma unroll
        for (int b = 0; b < WIDE_B; ++b)
            if (q0 + (uint32_t)b * NT + threadIdx.x < n) f(kk[b], cc[b]);
    }
}

// One unit's candidate list: LDS slots [0, own), then its workspace slots
// [own, n).  Only keys >= thr are visited as selectable.
struct WideSrc {
    static constexpr int SLOTS = 0;  // not held in registers
    uint32_t own, n, thr;
    const uint32_t* gkey;
    const uint32_t* gidx;
    template <class F>
    __device__ __forceinline__ void for_each(Smem& sm, F f) const {
        for (uint32_t q = threadIdx.x; q < own; q += NT) {
            const uint32_t key = sm.key[q];
            f(key >= thr, key, sm.idx[q]);
        }
        visit_global(gkey, gidx, own, n, [&](uint32_t key, uint32_t col) { f(key >= thr, key, col); });
    }
};

// The published lists of a split row's units: list q holds sm.seg_hi[q]
// entries at rkey / ridx + q * stride (every list fits its slots).
struct MergeSrc {
    static constexpr int SLOTS = 0;
    int lists;
    uint32_t thr, stride;
    const uint32_t* rkey;
    const uint32_t* ridx;
    template <class F>
    __device__ __forceinline__ void for_each(Smem& sm, F f) const {
        for (int q = 0; q < lists; ++q)
            visit_global(rkey + (size_t)q * stride, ridx + (size_t)q * stride, 0u, sm.seg_hi[q],
                         [&](uint32_t key, uint32_t col) { f(key >= thr, key, col); });
    }
};

// Every column of a window, read from the row on every visit: the exact
// fallback of the wide selections (one HBM pass per visit).
template <int DT, bool CANON>
struct RowSrc {
    static constexpr int SLOTS = 0;
    const typename Traits<DT>::raw_t* row;
    uint32_t n;
    template <class F>
    __device__ __forceinline__ void for_each(Smem&, F f) const {
        constexpr int B = 16;
        for (uint32_t c0 = 0; c0 < n; c0 += (uint32_t)NT * B) {
            uint32_t v[B];
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const uint32_t c = c0 + (uint32_t)b * NT + threadIdx.x;
                v[b] = (uint32_t)gload(row + (c < n ? c : 0u));
            }
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const uint32_t c = c0 + (uint32_t)b * NT + threadIdx.x;
                if (c < n) f(true, Keys<DT, CANON>::of(v[b]), c);
            }
        }
    }
};

// Deterministic-mode output of one entry at slot pos: the index through the
// policy and, for the varlen selection, the value -- the canonical key's own
// bits, or the element read back from the row where the key stands for
// several bit patterns (+-0, NaN).
template <int DT, class Policy>
__device__ __forceinline__ uint32_t ordered_raw(const Params& p, const typename Traits<DT>::raw_t* row,
                                                int32_t col, uint32_t key) {
    if constexpr (Policy::GATHERS) {
        return 0u;
    } else {
        if (col < 0) return Traits<DT>::PAD;
        if (p.out_vals && canon_special<DT>(key)) return (uint32_t)gload(row + col);
        return from_key<DT>(key);
    }
}

// Writes the entries (col, key) of slots [0, k) -- col < 0 for an empty slot --
// where entry(q) names slot q's entry, EJ slots per thread per round.  With
// a page table each round issues its table reads before any index store
// (a read placed after a store waits for it).
template <int DT, class Policy, class Entry>
__device__ __forceinline__ void emit_slots(const Params& p, int r, int64_t base,
                                           const typename Traits<DT>::raw_t* row, Entry entry) {
    constexpr int EJ = 8;
    const auto w = Policy::row(p, r, base);
    for (uint32_t q0 = 0; q0 < (uint32_t)p.k; q0 += (uint32_t)NT * EJ) {
        int32_t tv[EJ];
#pragma unroll
        for (int u = 0; u < EJ; ++u) {
            const uint32_t q = q0 + (uint32_t)u * NT + threadIdx.x;
            tv[u] = -1;
            if (q < (uint32_t)p.k) {
                int32_t col;
                uint32_t key;
                entry(q, col, key);
                if constexpr (Policy::GATHERS) {
                    Policy::put_raw(p, r, q, col);
                    tv[u] = Policy::translate(p, r, w, col);
                } else {
                    Policy::template emit<DT>(p, r, base, q, col, ordered_raw<DT, Policy>(p, row, col, key));
                }
            }
        }
        if constexpr (Policy::GATHERS) {
#pragma unroll
            for (int u = 0; u < EJ; ++u) {
                const uint32_t q = q0 + (uint32_t)u * NT + threadIdx.x;
                if (q < (uint32_t)p.k) Policy::put_idx(p, r, q, tv[u]);
            }
        }
    }
}

// Canonical order: sorts LDS slots [0, m) by key descending, then column
// ascending, and writes the first m through the policy, then -1 / pad values
// up to k.  The order is that of the 64-bit word (key << 32) | ~column, sorted
// descending by a bitonic network over P = NT * E words (E = 1, 2, 4 or 8, the
// smallest with P >= m; padding words are 0, below every entry).  The network
// is the form in which every step orders its pairs the same way: merge stage
// s (blocks of 2^(s+1) positions) first pairs position i with its mirror
// image i ^ (2^(s+1) - 1), then with i ^ 2^j for j = s-1 .. 0, and the lower
// position of each pair keeps the larger word.  Thread t keeps positions
// t*E .. t*E + E - 1 in registers: a pair inside the thread needs no
// exchange, a pair across lanes of one wave exchanges words by DPP (lanes
// 1 and 2 apart, mirrors of 4, 8 and 16 lanes) or ds_bpermute, and only
// pairs across waves pass through LDS.  The network is unrolled into straight
// code, so the words stay in registers without copies between steps; the
// kernel inlines it once, in its epilogue (defer_sort).
static_assert(CAP >= 2048, "a canonical-order sort of up to 2048 entries fits the candidate slots");
static_assert(NT == 256, "the register sort maps bits 6 and 7 of the thread index to waves");

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_word(uint64_t x) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)x, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(x >> 32), CTRL, 0xF, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t perm_word(uint64_t x, uint32_t addr) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute((int)addr, (int)(uint32_t)x);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute((int)addr, (int)(uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}

template <int E>
constexpr int log2_of() {
    return E == 1 ? 0 : E == 2 ? 1 : E == 4 ? 2 : 3;
}

// One step of the network.  MIR: pairs i with i ^ (2^(J+1) - 1), else with
// i ^ 2^J (J counts position bits: bits below log2 E select the register,
// the next 8 the thread).
template <int E, int J, bool MIR>
__device__ __forceinline__ void net_step(Smem& sm, uint64_t (&v)[E], uint32_t t) {
    constexpr int LE = log2_of<E>();
    if constexpr (J < LE) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (e & (1 << J)) continue;
            uint64_t& a = v[e];
            uint64_t& b = v[MIR ? e ^ ((2 << J) - 1) : e | (1 << J)];
            const bool swap = a < b;
            const uint64_t hi = swap ? b : a;
            b = swap ? a : b;
            a = hi;
        }
    } else {
        // the partner of (t, e) is (t ^ TM, MIR ? E-1-e : e); the lower
        // position is the one whose thread bit J - LE is clear
        constexpr uint32_t JT = (uint32_t)(J - LE);
        constexpr uint32_t TM = MIR ? (2u << JT) - 1u : 1u << JT;
        const bool keep_max = ((t >> JT) & 1u) == 0;
        uint64_t o[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint64_t x = v[MIR ? E - 1 - e : e];
            if constexpr (TM == 1) {
                o[e] = dpp_word<0xB1>(x);  // quad_perm 1,0,3,2
            } else if constexpr (TM == 2) {
                o[e] = dpp_word<0x4E>(x);  // quad_perm 2,3,0,1
            } else if constexpr (TM == 3) {
                o[e] = dpp_word<0x1B>(x);  // quad_perm 3,2,1,0
            } else if constexpr (TM == 7) {
                o[e] = dpp_word<0x141>(x);  // row_half_mirror
            } else if constexpr (TM == 15) {
                o[e] = dpp_word<0x140>(x);  // row_mirror
            } else if constexpr (TM < 64) {
                o[e] = perm_word(x, ((t & 63u) ^ TM) << 2);
            }
        }
        if constexpr (TM >= 64) {
            // across waves: every word goes through LDS at [e * NT + t]
            uint64_t* words = reinterpret_cast<uint64_t*>(sm.cand_words);
#pragma unroll
            for (int e = 0; e < E; ++e) words[e * NT + t] = v[e];
            lds_sync();
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = words[(MIR ? E - 1 - e : e) * NT + (t ^ TM)];
            lds_sync();
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const bool gt = v[e] > o[e];
            v[e] = gt == keep_max ? v[e] : o[e];
        }
    }
}

// Half-cleaner steps of strides 2^J .. 1.
template <int E, int J>
__device__ __forceinline__ void half_steps(Smem& sm, uint64_t (&v)[E], uint32_t t) {
    if constexpr (J >= 0) {
        net_step<E, J, false>(sm, v, t);
        half_steps<E, J - 1>(sm, v, t);
    }
}

// Merge stages S .. log2 P - 1, each its mirror step and then its
// half-cleaners.
template <int E, int S>
__device__ __forceinline__ void stages_from(Smem& sm, uint64_t (&v)[E], uint32_t t) {
    if constexpr (S < log2_of<E>() + 8) {
        net_step<E, S, true>(sm, v, t);
        half_steps<E, S - 1>(sm, v, t);
        stages_from<E, S + 1>(sm, v, t);
    }
}

template <int E>
__device__ __forceinline__ void sort_slots(Smem& sm, uint32_t m) {
    const uint32_t t = threadIdx.x;
    lds_sync();  // the slots were written by other threads
    uint64_t v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const uint32_t q = (uint32_t)e * NT + t;
        v[e] = q < m ? ((uint64_t)sm.key[q] << 32) | (uint32_t)~sm.idx[q] : 0ull;
    }
    lds_sync();  // the slots are read before the exchanges reuse their space
    stages_from<E, 0>(sm, v, threadIdx.x);
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const uint32_t q = t * (uint32_t)E + (uint32_t)e;
        sm.key[q] = (uint32_t)(v[e] >> 32);
        sm.idx[q] = ~(uint32_t)v[e];
    }
    lds_sync();
}

// Deterministic mode leaves the canonical sort to the kernel's epilogue, so
// that the network is inlined once per kernel: the m entries wait in LDS
// slots [0, m) of row r, whose window starts at `base`.
constexpr uint32_t NO_SORT = 0xFFFFFFFFu;

__device__ __forceinline__ void defer_sort(Smem& sm, int r, int64_t base, uint32_t m) {
    if (threadIdx.x == 0) {
        sm.sort_m = m;
        sm.sort_r = (uint32_t)r;
        sm.sort_base = (uint32_t)base;  // window starts lie in [0, width], width < 2^31
    }
}

template <int DT, class Policy>
__device__ __forceinline__ void sort_and_emit(Smem& sm, const Params& p, int r, int64_t base,
                                              const typename Traits<DT>::raw_t* row, uint32_t m) {
    if (m <= NT) {
        sort_slots<1>(sm, m);
    } else if (m <= 2 * NT) {
        sort_slots<2>(sm, m);
    } else if (m <= 4 * NT) {
        sort_slots<4>(sm, m);
    } else {
        sort_slots<8>(sm, m);
    }
    emit_slots<DT, Policy>(p, r, base, row, [&](uint32_t q, int32_t& col, uint32_t& key) {
        const bool in = q < m;
        col = in ? (int32_t)sm.idx[q] : -1;
        key = in ? sm.key[q] : 0u;
    });
}

// Deterministic mode for a row with more than k candidates: of the keys equal
// to the k-th key K, the k - gt with the smallest (ORDER_SMALL) or largest
// (ORDER_LARGE) columns are taken (a second exact select over their columns,
// which are distinct).  The k winners are gathered into LDS and sorted, or,
// with ORDER_NOSORT, written at once in no particular order.
template <int DT, class Policy, class Src>
__device__ __forceinline__ void ordered_emit(Smem& sm, const Params& p, int r, int64_t base,
                                             const typename Traits<DT>::raw_t* row,
                                             const Src& src, uint32_t K, uint32_t gt) {
    const uint32_t need_eq = (uint32_t)p.k - gt;
    const bool small = (p.order & 3) == ORDER_SMALL;
    uint32_t C, cgt;
    block_select_exact(
        sm,
        [&](auto f) {
            src.for_each(sm, [&](bool ok, uint32_t key, uint32_t col) {
                if (ok && key == K) f(small ? ~col : col);
            });
        },
        need_eq, C, cgt);
    if (threadIdx.x == 0) sm.cnt_a = 0;
    lds_sync();
    auto chosen = [&](bool ok, uint32_t key, uint32_t col) {
        return ok && (key > K || (key == K && (small ? ~col : col) >= C));
    };
    uint32_t nsel = 0;
    src.for_each(sm, [&](bool ok, uint32_t key, uint32_t col) { nsel += chosen(ok, key, col) ? 1u : 0u; });
    uint32_t o = wave_ticket_n(&sm.cnt_a, nsel);
    if (p.order & ORDER_NOSORT) {
        const auto w = Policy::row(p, r, base);
        src.for_each(sm, [&](bool ok, uint32_t key, uint32_t col) {
            if (chosen(ok, key, col)) {
                if constexpr (Policy::GATHERS) {
                    Policy::put_raw(p, r, o, (int32_t)col);
                    Policy::put_idx(p, r, o, Policy::translate(p, r, w, (int32_t)col));
                } else {
                    Policy::template emit<DT>(p, r, base, o, (int32_t)col,
                                              ordered_raw<DT, Policy>(p, row, (int32_t)col, key));
                }
                ++o;
            }
        });
        return;
    }
    src.for_each(sm, [&](bool ok, uint32_t key, uint32_t col) {
        if (chosen(ok, key, col)) {
            sm.key[o] = key;
            sm.idx[o] = col;
            ++o;
        }
    });
    defer_sort(sm, r, base, (uint32_t)p.k);
}

// Selects the top k of `src` (which must hold at least k entries and contain
// a top-k of the row) and writes them through the policy.
template <int DT, class Policy, class Src>
__device__ __forceinline__ void select_and_emit(Smem& sm, const Params& p, int r, int64_t base,
                                                const typename Traits<DT>::raw_t* row, const Src& src) {
    VTS_STAMP(8);
    uint32_t K, gt;
    const auto keys = [&](auto f) {
        src.for_each(sm, [&](bool ok, uint32_t key, uint32_t) {
            if (ok) f(key);
        });
    };
    if constexpr (Policy::ORDERED) {
        block_select_exact(sm, keys, (uint32_t)p.k, K, gt);
        VTS_STAMP(9);
        ordered_emit<DT, Policy>(sm, p, r, base, row, src, K, gt);
        return;
    }
    // The top k: the gt keys above Ktop and the k - gt first keys in [K,
    // Ktop] (every key of that range when the selection ended on a digit
    // that completes the rank; otherwise K == Ktop, the k-th key).  Only
    // 32-bit keys take the early end: it saves their third pass, while
    // 16-bit keys need two passes at most.
    constexpr bool RANGE = Traits<DT>::BITS > 16;
    uint32_t Ktop;
    if constexpr (RANGE) {
        block_select_range(sm, keys, (uint32_t)p.k, K, Ktop, gt);
    } else {
        block_select_exact(sm, keys, (uint32_t)p.k, K, gt);
        Ktop = K;
    }
    VTS_STAMP(9);
    const uint32_t span = Ktop - K;
    const auto above = [&](uint32_t key) { return key > Ktop; };
    const auto at = [&](uint32_t key) {  // key in [K, Ktop]
        if constexpr (RANGE) return key - K <= span;
        else return key == K;
    };
    const uint32_t need_eq = (uint32_t)p.k - gt;
    // With a page table whose entries for the row's window fit the staging
    // area (free now that the selections are done), they go to LDS and the
    // translation reads no global memory between the output stores.  The
    // first TJ * NT entries are read here and land while the outputs are
    // counted; the rest of a longer window are read after the count.  (Read
    // before the selection instead, they made it slower by as much as they
    // saved here.)
    constexpr int TJ = 5;  // 1280 entries: a 65536-column window of 64-column pages
    [[maybe_unused]] uint32_t tl[TJ];
    uint32_t np = 0;
    [[maybe_unused]] StagedTable stg{};
    if constexpr (Policy::GATHERS && Src::SLOTS > 0) {
        np = Policy::table_pages(p, (uint32_t)__builtin_amdgcn_readfirstlane((int)sm.row_n));
        if (np > (uint32_t)TABLE_WORDS) np = 0;
        if (np) {
            const auto w = Policy::row(p, r, base);
            stg = Policy::staged(p, w, sm.table, np);
            Policy::template table_fetch<TJ>(p, r, w, stg, tl);
        }
    }
    if (threadIdx.x == 0) {
        sm.cnt_a = 0;
        sm.cnt_b = 0;
    }
    lds_sync();
    // Each thread counts its keys above the range and in it; one bit-sliced
    // wave prefix and one LDS ticket per wave and list give every thread its
    // first output slots, and its keys are written in order from there.
    uint32_t ngt = 0, neq = 0;
    src.for_each(sm, [&](bool ok, uint32_t key, uint32_t) {
        ngt += (ok && above(key)) ? 1u : 0u;
        neq += (ok && at(key)) ? 1u : 0u;
    });
    // (a wide source can give a thread more entries than wave_ticket_n counts)
    uint32_t og, oe;
    if constexpr (Src::SLOTS > 0) {
        og = wave_ticket_n(&sm.cnt_a, ngt);
        oe = wave_ticket_n(&sm.cnt_b, neq);
    } else {
        og = wave_ticket_any(&sm.cnt_a, ngt);
        oe = wave_ticket_any(&sm.cnt_b, neq);
    }
    VTS_STAMP(13);
    if constexpr (Policy::GATHERS) {
        const auto w = Policy::row(p, r, base);
        // (sources held in registers only; a wide source translates inline)
        bool ahead = false;
        if constexpr (Src::SLOTS > 0) ahead = Policy::gathers(p);
        if (np) {
#pragma unroll
            for (int u = 0; u < TJ; ++u) {
                const uint32_t j = (uint32_t)u * NT + threadIdx.x;
                if (j < np) sm.table[j] = tl[u];
            }
            for (uint32_t j = (uint32_t)TJ * NT + threadIdx.x; j < np; j += NT)
                sm.table[j] = j >= stg.jlo && j < stg.jhi ? (uint32_t)gload(p.pt + (int64_t)r * p.pt_stride + w.start + j) : 0u;
            lds_sync();
        }
        VTS_STAMP(14);
        if (ahead) {
          if constexpr (Src::SLOTS > 0) {
            // Every table read of the thread is issued before its first output
            // index store.  Placed after a store, a read would wait for it (the
            // compiler cannot rule out that they overlap, and loads and stores
            // share one completion counter), one memory round trip per register.
            // The first pass also writes the raw indices, so the registers that
            // held them take the translated ones and the pass adds none.
            const OutRow o = Policy::template out_row<DT>(p, r);
            auto two_passes = [&](auto translate) {
                const uint32_t og0 = og, oe0 = oe;
                int32_t tv[Src::SLOTS];
                src.for_each_slot([&](int j, bool ok, uint32_t key, uint32_t col) {
                    const bool isgt = ok && above(key), iseq = ok && at(key);
                    const uint32_t pos = isgt ? og : gt + oe;
                    tv[j] = -1;
                    if (isgt || (iseq && oe < need_eq)) {
                        Policy::put_raw(o, pos, (int32_t)col);
                        tv[j] = translate((int32_t)col);
                    }
                    og += isgt ? 1u : 0u;
                    oe += iseq ? 1u : 0u;
                });
                og = og0;
                oe = oe0;
                src.for_each_slot([&](int j, bool ok, uint32_t key, uint32_t) {
                    const bool isgt = ok && above(key), iseq = ok && at(key);
                    const uint32_t pos = isgt ? og : gt + oe;
                    if (isgt || (iseq && oe < need_eq)) Policy::put_idx(o, pos, tv[j]);
                    og += isgt ? 1u : 0u;
                    oe += iseq ? 1u : 0u;
                });
            };
            if (np) {
                // The translation reads LDS only.  Every register's entry is
                // read first, without a branch (a read inside each store's
                // condition would wait for its own round trip), then the
                // stores.
                int32_t tv[Src::SLOTS];
                src.for_each_slot([&](int j, bool, uint32_t, uint32_t col) {
                    tv[j] = Policy::translate_staged(stg, col);
                });
                src.for_each_slot([&](int j, bool ok, uint32_t key, uint32_t col) {
                    const bool isgt = ok && above(key), iseq = ok && at(key);
                    const uint32_t pos = isgt ? og : gt + oe;
                    if (isgt || (iseq && oe < need_eq)) {
                        Policy::put_raw(o, pos, (int32_t)col);
                        Policy::put_idx(o, pos, tv[j]);
                    }
                    og += isgt ? 1u : 0u;
                    oe += iseq ? 1u : 0u;
                });
            } else {
                two_passes([&](int32_t col) { return Policy::translate(p, r, w, col); });
            }
          }
        } else {
            const OutRow o = Policy::template out_row<DT>(p, r);
            src.for_each(sm, [&](bool ok, uint32_t key, uint32_t col) {
                const bool isgt = ok && above(key), iseq = ok && at(key);
                const uint32_t pos = isgt ? og : gt + oe;
                if (isgt || (iseq && oe < need_eq)) {
                    Policy::put_raw(o, pos, (int32_t)col);
                    Policy::put_idx(o, pos, Policy::translate(p, r, w, (int32_t)col));
                }
                og += isgt ? 1u : 0u;
                oe += iseq ? 1u : 0u;
            });
        }
    } else {
        const OutRow o = Policy::template out_row<DT>(p, r);
        src.for_each(sm, [&](bool ok, uint32_t key, uint32_t col) {
            const bool isgt = ok && above(key), iseq = ok && at(key);
            const uint32_t pos = isgt ? og : gt + oe;
            if (isgt || (iseq && oe < need_eq))
                Policy::template put<DT>(o, pos, (int32_t)col, from_key<DT>(key));
            og += isgt ? 1u : 0u;
            oe += iseq ? 1u : 0u;
        });
    }
}

// A short row (n <= k): the identity, then -1 (and the values, or padding).
// With a page table each round of SHORT_J slots per thread issues its table
// reads before any index store.
constexpr int SHORT_J = 8;

template <int DT, class Policy>
__device__ __forceinline__ void short_row(const Params& p, int r, int64_t base, int64_t n,
                          const typename Traits<DT>::raw_t* row) {
    if constexpr (Policy::GATHERS) {
        // as in select_and_emit: the table reads before the index stores
        const auto w = Policy::row(p, r, base);
        for (int j0 = 0; j0 < p.k; j0 += SHORT_J * NT) {
            int32_t tv[SHORT_J];
#pragma unroll
            for (int u = 0; u < SHORT_J; ++u) {
                const int j = j0 + u * NT + (int)threadIdx.x;
                tv[u] = -1;
                if (j < p.k) {
                    Policy::put_raw(p, r, (uint32_t)j, j < n ? j : -1);
                    if (j < n) tv[u] = Policy::translate(p, r, w, j);
                }
            }
#pragma unroll
            for (int u = 0; u < SHORT_J; ++u) {
                const int j = j0 + u * NT + (int)threadIdx.x;
                if (j < p.k) Policy::put_idx(p, r, (uint32_t)j, tv[u]);
            }
        }
    } else {
        for (int j = threadIdx.x; j < p.k; j += NT) {
            const bool in = j < n;
            Policy::template emit<DT>(p, r, base, (uint32_t)j, in ? j : -1,
                                      in ? (uint32_t)gload(row + j) : Traits<DT>::PAD);
        }
    }
}

// Whole-row re-selection with the compaction filter (threshold: everything).
template <int DT, class Policy>
__device__ __forceinline__ void whole_row(Smem& sm, const Params& p, int r, int64_t base, int64_t n,
                          const typename Traits<DT>::raw_t* row) {
    const Slice s = make_slice<DT>(row, n, 0, 1);
    careful_filter<DT>(sm, p, row, s, make_thr<Policy::ORDERED>(p, 0u));
    __syncthreads();
    const uint32_t cand = sm.cand_n;
    __syncthreads();
    select_and_emit<DT, Policy>(sm, p, r, base, row, LdsSrc<ONCHIP_J>(sm, cand));
}

// Length-balanced placement of rows (one workgroup per row, R = 256 * s rows,
// 2 <= s <= 4).  Rows ordered by valid length -- longest first, in 32 length
// buckets, by row index within a bucket -- are dealt to compute units in a
// snake: the workgroups that share compute unit g (see BALANCE_CUS) take ranks
// g, 511 - g, 512 + g, 1023 - g, ..., so every unit's rows add up to about the
// same number of columns and no unit is left with only long rows.  Every
// workgroup derives the same ranking from the row lengths, and the map from
// blocks to ranks is a bijection, so each row is taken exactly once; the
// placement only changes speed.  The row's window comes back in base / n;
// c = 0 and eff = 1 (one unit per row).  Every thread must call it.
template <class Policy>
__device__ __forceinline__ int balanced_row(Smem& sm, const Params& p, uint32_t bid,
                                            int64_t& base, int64_t& n, int& c, int& eff) {
    constexpr int NB = 32;
    constexpr int MAXPER = 4;  // rows per thread (R <= 4 * NT)
    const int per = p.num_rows / NT;
    // scratch in the histogram, which is cleared before its first use
    uint32_t* cnt = sm.hist;          // NB bucket counts
    uint32_t* wcnt = sm.hist + 2 * NB;  // per chunk and wave: rows of the wanted bucket
    uint32_t bk[MAXPER];
    uint32_t wb[MAXPER], wn[MAXPER];  // windows of this thread's rows (< 2^31)
    // every row's loads first (their latency is the cost here), then the lengths
    typename Policy::Raw raw[MAXPER];
#pragma unroll
    for (int i = 0; i < MAXPER; ++i)
        raw[i] = Policy::fetch(p, i < per ? (int)threadIdx.x + i * NT : 0);
    const float scale = (float)NB / (float)(p.width + 1);
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
        int64_t b, n;
        Policy::finish(p, (int)threadIdx.x + i * NT, raw[i], b, n);
        wb[i] = (uint32_t)b;
        wn[i] = (uint32_t)n;
        uint32_t q = (uint32_t)((float)n * scale);  // 0..NB-1, longer rows higher
        q = q > NB - 1 ? NB - 1 : q;
        bk[i] = i < per ? NB - 1 - q : (uint32_t)NB;  // 0: longest; NB: no row
    }
    if (threadIdx.x < NB) cnt[threadIdx.x] = 0;
    if (threadIdx.x == 0) sm.total = 0xFFFFFFFFu;
    lds_sync();
#pragma unroll
    for (int i = 0; i < MAXPER; ++i)
        if (i < per) atomicAdd(&cnt[bk[i]], 1u);
    lds_sync();
    // Workgroup bid lands on compute unit k % 32 of XCD x (bid = 8k + x),
    // numbered g = 32 x + k % 32, and in round j = k / 32 it takes the row of
    // rank j * 256 + g (even rounds) or j * 256 + 255 - g (odd rounds; rank 0:
    // the longest), a serpentine that gives every compute unit a long row and
    // a short one.
    static_assert(BALANCE_CUS == 256 && BALANCE_XCDS == 8, "8 XCDs of 32 compute units");
    c = 0;
    eff = 1;
    const uint32_t x = bid % BALANCE_XCDS, k = bid / BALANCE_XCDS;
    const uint32_t g = x * BALANCE_CUS_PER_XCD + k % BALANCE_CUS_PER_XCD;
    const uint32_t j = k / BALANCE_CUS_PER_XCD;
    const uint32_t rank = j * BALANCE_CUS + ((j & 1u) ? BALANCE_CUS - 1 - g : g);
    // bucket holding the rank and the rank within it (the same in every
    // thread): lane b scans bucket b's count, the first lane whose running
    // total passes the rank names it
    static_assert(NB <= 64, "one bucket per lane");
    const uint32_t lb = lane_id();
    const uint32_t cb = lb < (uint32_t)NB ? cnt[lb] : 0u;
    const uint32_t incl = wave_scan(cb, 0u, OpAdd());
    const uint64_t past = ballot(lb < (uint32_t)NB && incl > rank);
    const uint32_t want = past ? (uint32_t)__builtin_ctzll(past) : (uint32_t)NB;
    const uint32_t m =
        past ? rank - (uint32_t)__builtin_amdgcn_readlane((int)(incl - cb), (int)want) : 0u;
    // The m-th row of that bucket in row order; row i * NT + t is thread t's
    // bk[i].  One ballot per chunk i, all counts published at once.
    const uint32_t w = threadIdx.x >> 6;
    uint64_t mask[MAXPER];
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
        mask[i] = ballot(bk[i] == want);
        if (i < per && lane_id() == 0) wcnt[i * WAVES + w] = (uint32_t)__popcll(mask[i]);
    }
    lds_sync();
    uint32_t before = 0;  // rows of the bucket before chunk i, wave w
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
        if (i >= per) break;
        uint32_t mine = 0, chunk = 0;
#pragma unroll
        for (int v = 0; v < WAVES; ++v) {
            const uint32_t c = wcnt[i * WAVES + v];
            mine += (uint32_t)v < w ? c : 0u;
            chunk += c;
        }
        const uint32_t r0 = before + mine + mbcnt(mask[i]);
        if (bk[i] == want && r0 == m) {
            sm.total = (uint32_t)((int)threadIdx.x + i * NT);
            sm.win_base = wb[i];
            sm.win_n = wn[i];
        }
        before += chunk;
    }
    lds_sync();
    const int row = (int)sm.total;
    base = sm.win_base;
    n = sm.win_n;
    lds_sync();  // sm.total and the histogram are rewritten later
    if (row >= 0 && row < p.num_rows) return row;
    const int r = (int)(bid % (uint32_t)p.num_rows);  // not reached: the map is a bijection
    Policy::window(p, r, base, n);
    return r;
}

// Length-balanced units for a batch of R = 2 * BALANCE_CUS rows, launched
// with 2 * R workgroups (four per compute unit).  A workgroup's stream is
// capped by the memory requests its compute unit keeps in flight, so a row
// far longer than the others would finish long after them; here every row is
// cut into e = min(EMAX_UNITS, ceil(n / U)) equal units, where U is about the
// batch's columns per compute unit (and at least split_cols), and the units --
// ranked by size, longest first, in NB buckets over [0, U], by row index
// within a bucket, each row covering e consecutive ranks -- are dealt to the
// compute units in serpentine rounds as in balanced_row (ranks g, 511 - g,
// 512 + g, 1023 - g on compute unit g, numbered g = 8 (k % 32) + x for block
// 8k + x so that consecutive ranks alternate over the XCDs).  U bounds the
// units at R + BALANCE_CUS <= 2 R; the ranks past them have nothing to do.
// Row r's units are numbered ubase(r) + c, c < e, where ubase(r) counts the
// units of the rows before r: they index the workspace lists and counts, and
// the row's ticket counts e.  Every workgroup derives the same units from
// the same integers, so each unit is taken exactly once.  Returns the row;
// base / n its window, c the unit (-1: nothing to do), eff = e, ubase.
// Every thread must call it.
constexpr int EMAX_UNITS = 8;

template <class Policy>
__device__ __forceinline__ int placed_unit(Smem& sm, const Params& p, uint32_t bid, int64_t& base,
                                           int64_t& n, int& c, int& eff, uint32_t& ubase) {
    constexpr int NB = 32;
    constexpr int MAXPER = 2;  // rows per thread: R = 2 * NT
    static_assert(2 * BALANCE_CUS == MAXPER * NT && BALANCE_CUS == 256 && BALANCE_XCDS == 8,
                  "two rows per thread, four workgroups per compute unit");
    static_assert(EMAX_UNITS <= MAX_SPLIT, "a row's lists fit the merge");
    // scratch in the histogram, which is cleared before its first use
    uint32_t* cnt = sm.hist;                          // NB bucket unit counts
    uint32_t* ktot = sm.hist + NB;                    // every row's valid columns / 1024
    uint32_t* wcnt = sm.hist + 2 * NB;                // per chunk, wave: units of the wanted bucket
    uint32_t* wall = wcnt + MAXPER * WAVES;           // per chunk, wave: units of every row
    uint32_t* found = wall + MAXPER * WAVES;          // the unit's row, window, c, e, ubase
    static_assert(2 * NB + 2 * MAXPER * WAVES + 6 <= HIST_WORDS, "scratch fits the histogram");
    uint32_t wb[MAXPER], wn[MAXPER], we[MAXPER], bk[MAXPER];
    typename Policy::Raw raw[MAXPER];
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) raw[i] = Policy::fetch(p, (int)threadIdx.x + i * NT);
    uint32_t ksum = 0;  // this thread's rows: valid columns / 1024 (exact)
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
        int64_t b, m;
        Policy::finish(p, (int)threadIdx.x + i * NT, raw[i], b, m);
        wb[i] = (uint32_t)b;
        wn[i] = (uint32_t)m;
        ksum += wn[i] >> 10;
    }
    if (threadIdx.x < NB) cnt[threadIdx.x] = 0;
    if (threadIdx.x == 0) {
        *ktot = 0;
        found[0] = 0xFFFFFFFFu;
    }
    lds_sync();
    {
        const uint32_t wk = wave_scan(ksum, 0u, OpAdd());  // < 2^31: R * width / 1024
        if (lane_id() == 63) atomicAdd(ktot, wk);
    }
    lds_sync();
    // U >= (the batch's columns) / BALANCE_CUS: the columns are at most
    // 1024 ktot + 1023 R, so the units' sum of n / U is at most BALANCE_CUS and
    // there are at most R + BALANCE_CUS units.  U <= width < 2^31.
    const uint64_t u64 = 4ull * *ktot + 4ull * (uint64_t)p.num_rows;
    uint32_t U = u64 < (uint64_t)p.width ? (uint32_t)u64 : (uint32_t)p.width;
    U = U > (uint32_t)p.split_cols ? U : (uint32_t)p.split_cols;
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
        uint32_t e = (wn[i] + U - 1) / U;  // < 2^32: wn, U < 2^31
        e = e < 1u ? 1u : (e > (uint32_t)EMAX_UNITS ? (uint32_t)EMAX_UNITS : e);
        we[i] = e;
        const uint32_t sz = wn[i] / e;  // a unit's columns
        uint64_t q = (uint64_t)sz * NB / ((uint64_t)U + 1u);  // 0..NB-1, larger units higher
        q = q > NB - 1 ? NB - 1 : q;
        bk[i] = NB - 1 - (uint32_t)q;  // 0: largest
        atomicAdd(&cnt[bk[i]], e);
    }
    lds_sync();
    const uint32_t x = bid % BALANCE_XCDS, k = bid / BALANCE_XCDS;
    const uint32_t g = (k % BALANCE_CUS_PER_XCD) * BALANCE_XCDS + x;
    const uint32_t j = k / BALANCE_CUS_PER_XCD;
    const uint32_t rank = j * BALANCE_CUS + ((j & 1u) ? BALANCE_CUS - 1 - g : g);
    // bucket holding the rank and the rank within it (the same in every
    // thread): lane b scans bucket b's count
    const uint32_t lb = lane_id();
    const uint32_t cb = lb < (uint32_t)NB ? cnt[lb] : 0u;
    const uint32_t incl = wave_scan(cb, 0u, OpAdd());
    const uint64_t past = ballot(lb < (uint32_t)NB && incl > rank);
    if (past == 0) {  // (uniform) past the last unit
        lds_sync();   // every thread has read the counts
        c = -1;
        eff = 1;
        base = 0;
        n = 0;
        ubase = 0;
        return 0;
    }
    const uint32_t want = (uint32_t)__builtin_ctzll(past);
    const uint32_t m = rank - (uint32_t)__builtin_amdgcn_readlane((int)(incl - cb), (int)want);
    // Rows in row order (row i * NT + t is thread t's chunk i): wave prefix
    // sums of their unit counts, in the wanted bucket and over every row.
    const uint32_t w = threadIdx.x >> 6;
    uint32_t exw[MAXPER], exa[MAXPER];
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
        const uint32_t vw = bk[i] == want ? we[i] : 0u;
        const uint32_t iw = wave_scan(vw, 0u, OpAdd());
        const uint32_t ia = wave_scan(we[i], 0u, OpAdd());
        exw[i] = iw - vw;
        exa[i] = ia - we[i];
        if (lane_id() == 63) {
            wcnt[i * WAVES + w] = iw;
            wall[i * WAVES + w] = ia;
        }
    }
    lds_sync();
    uint32_t before = 0, beforea = 0;  // units before chunk i: wanted bucket / every row
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
        uint32_t mine = 0, chunk = 0, minea = 0, chunka = 0;
#pragma unroll
        for (int v = 0; v < WAVES; ++v) {
            const uint32_t cw = wcnt[i * WAVES + v], ca = wall[i * WAVES + v];
            mine += (uint32_t)v < w ? cw : 0u;
            chunk += cw;
            minea += (uint32_t)v < w ? ca : 0u;
            chunka += ca;
        }
        const uint32_t r0 = before + mine + exw[i];
        if (bk[i] == want && m >= r0 && m < r0 + we[i]) {
            found[0] = threadIdx.x + (uint32_t)i * NT;
            found[1] = wb[i];
            found[2] = wn[i];
            found[3] = m - r0;
            found[4] = we[i];
            found[5] = beforea + minea + exa[i];
        }
        before += chunk;
        beforea += chunka;
    }
    lds_sync();
    const int row = (int)found[0];
    base = found[1];
    n = found[2];
    c = (int)found[3];
    eff = (int)found[4];
    ubase = found[5];
    lds_sync();  // the histogram is rewritten later
    if (row >= 0 && row < p.num_rows) return row;
    c = -1;  // not reached: every rank below the unit count names a unit
    return 0;
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

// WIDE: the instantiation for top_k > 2048 (unordered policies only), whose
// candidate lists outgrow the registers; see the WIDE branch below.  HINT:
// the instantiation for calls with a hint (varlen, top_k <= 2048), whose
// safe rung is also bounded below by the hint rung.
template <int DT, class Policy, bool WIDE, bool HINT>
__device__ __forceinline__ void topk_unit(Smem& sm, const Params& p, uint32_t bid, uint32_t unit) {
    using raw_t = typename Traits<DT>::raw_t;
    constexpr bool ORD = Policy::ORDERED;  // deterministic mode: canonical keys
#ifdef VTS_PHASE_STAMPS
    // the workgroup's slot (thread 0 alone writes and reads it), kept when a
    // split row renumbers the unit
    if (threadIdx.x == 0) sm.stamp_unit = unit;
#endif
    VTS_STAMP(0);
    // The row and its window are the same in every lane, but they arrive
    // through LDS and vector loads; readfirstlane puts them in scalar
    // registers, so the stream's buffer offsets are scalar and its loads need
    // no per-lane loop.
    int64_t base, n;
    int r, c = 0, beff = 1;
    uint32_t ubase = 0;  // (units) the row's first unit
    if (p.balance) {
        if (p.helpers)
            r = placed_unit<Policy>(sm, p, bid, base, n, c, beff, ubase);
        else
            r = balanced_row<Policy>(sm, p, bid, base, n, c, beff);
        c = __builtin_amdgcn_readfirstlane(c);
        if (c < 0) return;  // a workgroup past the last unit
        ubase = (uint32_t)__builtin_amdgcn_readfirstlane((int)ubase);
    } else {
        r = (int)(unit / (uint32_t)p.nsplit);
        Policy::window(p, r, base, n);
    }
    r = __builtin_amdgcn_readfirstlane(r);
    if (!p.balance) c = (int)(unit - (uint32_t)r * (uint32_t)p.nsplit);
    // window starts and lengths lie in [0, width], width < 2^31
    base = __builtin_amdgcn_readfirstlane((int)base);
    n = __builtin_amdgcn_readfirstlane((int)n);
    VTS_STAMP(1);
    VTS_STAMP_ID(r, n);
    if (threadIdx.x == 0) sm.row_n = (uint32_t)n;
    const raw_t* row = static_cast<const raw_t*>(p.x) + (int64_t)r * p.row_stride + base;
    if (n <= p.k) {
        if (c == 0) {
            if (ORD && !(p.order & ORDER_NOSORT)) {
                // every column is selected; canonical order sorts them
                lds_sync();
                for (int j = threadIdx.x; j < n; j += NT) {
                    sm.key[j] = Keys<DT, ORD>::of((uint32_t)gload(row + j));
                    sm.idx[j] = (uint32_t)j;
                }
                defer_sort(sm, r, base, (uint32_t)n);
            } else {
                short_row<DT, Policy>(p, r, base, n, row);
            }
        }
        VTS_STAMP(4);
        return;
    }
    int64_t eff64 = (n + p.min_chunk - 1) / p.min_chunk;
    if (eff64 > p.nsplit) eff64 = p.nsplit;
    if (eff64 < 1) eff64 = 1;
    const int eff = p.balance ? __builtin_amdgcn_readfirstlane(beff) : (int)eff64;
    if (c >= eff) return;
    // The row's units, which the split-row merge reads: ubase + c with the
    // length-balanced units, r * nsplit + c otherwise (a placed row of whole
    // units keeps its workgroup's own unit).
    const uint32_t unit0 = p.helpers ? ubase : (uint32_t)r * (uint32_t)p.nsplit;
    if (p.helpers) unit = ubase + (uint32_t)c;

    const Slice s = make_slice<DT>(row, n, c, eff);
    uint32_t* gkey = p.ws_key + (size_t)unit * (uint32_t)p.ws_slots;
    uint32_t* gidx = p.ws_idx + (size_t)unit * (uint32_t)p.ws_slots;
    const Buf B{gkey, gidx, (uint32_t)p.lds_cap, (uint32_t)p.hi_cap};
    // body vectors of this unit, relative indexing (32-bit)
    const u32x4* vb = reinterpret_cast<const u32x4*>(row + s.h) + s.v0;
    const uint32_t nvec = (uint32_t)(s.v1 - s.v0);
    const uint32_t col0 = (uint32_t)(s.h + s.v0 * Traits<DT>::VE);
    constexpr int U = Traits<DT>::U;

    // The sample's loads go out first; the first streaming step's follow once
    // the sample has landed and stay in flight while the rungs are computed.
    // With a hint, the hinted columns are loaded before the sample and the
    // row's values at them right after it (those reads need the columns).
    static_assert(!(HINT && (WIDE || Policy::GATHERS)), "hints serve the varlen selection");
    HintReads<DT> H;
    if constexpr (HINT) hint_cols(p, r / p.next_n, H.col);
    Sample<DT> S;
    sample_load<DT>(row, n, spread_hash((uint32_t)r), S);
    if constexpr (HINT) hint_reads<DT>(row, n, H);
    u32x4 RA[U], RB[U];
    static_assert(!(WIDE && ORD), "the deterministic mode is limited to top_k <= 2048");
    bool refiltered = !WIDE && p.force_path == FORCE_CAREFUL;
    // (always issued, also where the careful filter will ignore it: straight-line
    // code keeps the wait counts exact)
    const __amdgpu_buffer_rsrc_t rs = body_rsrc(vb, nvec * 16u);
    constexpr uint32_t STEP = (uint32_t)NT * U;
    StepOrder order;
    order.nsteps = (nvec + STEP - 1) / STEP;
    order.rot = order.nsteps > 1
                    ? (uint32_t)(((uint64_t)spread_hash(unit) * order.nsteps) >> 32)
                    : 0u;
    if (threadIdx.x == 0) {
        sm.cand_n = 0;
        sm.up_n = 0;
    }
    hist_clear(sm);    // every select leaves the histogram zeroed again
    spread_clear(sm);  // the sample select's first-pass copies
    if constexpr (HINT) hint_map_clear(sm);
    lds_sync();        // the loads stay in flight
    // A row that the sample read whole and that fits the on-chip candidate
    // slots is selected directly: its first unit puts every column in the
    // slot of its column (a second, cache-hot read of at most CAP elements)
    // and selects from there -- no rungs, no stream; the row's other units,
    // if any, have nothing to do.
    const bool direct = S.whole && n <= (int64_t)B.lds_cap && p.force_path == FORCE_NONE;
    if (direct) {
        if (c != 0) return;
        for (uint32_t col = threadIdx.x; col < (uint32_t)n; col += NT) {
            sm.key[col] = Keys<DT, ORD>::of(gload(row + col));
            sm.idx[col] = col;
        }
        __syncthreads();
    }
    Rungs G{0u, 0u};
    if (!direct) {
        uint32_t TH = 0u;
        if constexpr (HINT) {
            if (!S.whole) {  // (a whole-row sample is exact already)
                TH = hint_rung<DT>(sm, p, n, H);
                spread_clear(sm);
                lds_sync();
            }
        }
        G = sample_rungs<DT>(sm, p, n, S, [&]() {
            VTS_STAMP(15);
            load_step(RA, rs, order.first(0, STEP));
        });
        if constexpr (HINT) {  // both rungs are lower bounds of the k-th largest key
            G.T = G.T > TH ? G.T : TH;
            G.T2 = G.T2 > TH ? G.T2 : TH;
        }
        if constexpr (ORD) {  // rungs the canonical keys and the raw-bit tests agree on
            G.T = canon_floor<DT>(G.T);
            G.T2 = canon_floor<DT>(G.T2);
        }
    }
    VTS_STAMP(2);

    uint32_t nh = 0, nup = 0;  // candidates (keys >= T), of which keys >= T2
    if (direct) {
        nh = (uint32_t)n;  // every column, on chip
    } else if (!refiltered) {
        filter_scalars<DT, ORD>(sm, B, row, s.s0, s.s1, G);
        constexpr uint32_t SIGN = Traits<DT>::BITS == 32 ? 0x80000000u : 0x8000u;
        if (nvec == 0) {
        } else if (G.T & G.T2 & SIGN) {  // both rungs >= +0: raw-bit compares
            stream_unit<DT, true, ORD>(sm, B, RA, RB, rs, nvec, col0, G, order);
        } else {
            stream_unit<DT, false, ORD>(sm, B, RA, RB, rs, nvec, col0, G, order);
        }
        filter_scalars<DT, ORD>(sm, B, row, s.t0, s.t1, G);
        __syncthreads();  // also completes the workspace stores of every thread
        nh = sm.cand_n;
        nup = sm.up_n;
        VTS_STAMP(3);
        hist_clear(sm);  // the staging queues overlaid the histogram
        lds_sync();      // everyone has read the counts before they can change
        if (!WIDE && nh > B.hi_cap) {  // slots ran out: re-filter with compaction
            if (threadIdx.x == 0) gatomic_add(p.ws_stats + 0, 1u);
            refiltered = true;
        }
    }
    if (refiltered) {
        careful_filter<DT>(sm, p, row, s, make_thr<ORD>(p, G.T));
        __syncthreads();
        nh = sm.cand_n;  // every candidate is on chip now
        nup = 0;
        __syncthreads();
    }
    if constexpr (WIDE) {
        // Wide selections keep every candidate (LDS slots, then the unit's
        // workspace slots: hi_cap covers twice top_k) and select from there.
        // Exactness still rests on the counts: fewer than k candidates, a
        // list past its slots or a forced path re-select the row exactly with
        // radix passes over the row itself (RowSrc).
        const bool over = nh > B.hi_cap;
        const bool forced = p.force_path != FORCE_NONE;
        const uint32_t own = nh < B.lds_cap ? nh : B.lds_cap;
        const bool upper = nup >= (uint32_t)p.k;
        if (eff == 1 || direct) {
            if (nh < (uint32_t)p.k || over || forced) {
                if (threadIdx.x == 0 && (nh < (uint32_t)p.k || over))
                    gatomic_add(p.ws_stats + (over ? 0 : 1), 1u);
                __syncthreads();
                select_and_emit<DT, Policy>(sm, p, r, base, row, RowSrc<DT, ORD>{row, (uint32_t)n});
                VTS_STAMP(4);
                return;
            }
            if (threadIdx.x == 0 && !upper) gatomic_add(p.ws_stats + 3, 1u);
            const uint32_t thr = upper ? G.T2 : 0u;
            if (nh <= own) {
                select_and_emit<DT, Policy>(sm, p, r, base, row, LdsSrc<ONCHIP_J>(sm, nh, thr));
            } else {
                if (threadIdx.x == 0) gatomic_add(p.ws_stats + 2, 1u);
                select_and_emit<DT, Policy>(sm, p, r, base, row, WideSrc{own, nh, thr, gkey, gidx});
            }
            VTS_STAMP(4);
            return;
        }
        // split row: publish the on-chip part behind which the spill already
        // sits, the counts (bit 31 of the second: the list outgrew its slots),
        // then the ticket; the last unit selects over all the lists
        for (uint32_t q = threadIdx.x; q < own; q += NT) {
            gstore(gkey + q, sm.key[q]);
            gstore(gidx + q, sm.idx[q]);
        }
        if (threadIdx.x == 0) {
            gstore(p.ws_count + unit, over ? (uint32_t)B.hi_cap : nh);
            gstore(p.ws_count_up + unit, nup | (over ? 0x80000000u : 0u));
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            const uint32_t old = __hip_atomic_fetch_add((VTS_GLOBAL uint32_t*)(p.ws_ticket + r), 1u,
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const bool last = old == (uint32_t)eff - 1u;
            if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            sm.flag = last ? 1u : 0u;
        }
        __syncthreads();
        VTS_STAMP(5);
        if (sm.flag == 0) return;
        if (threadIdx.x < (unsigned)eff) {
            sm.seg_hi[threadIdx.x] = gload(p.ws_count + unit0 + threadIdx.x);
            sm.seg_lo[threadIdx.x] = gload(p.ws_count_up + unit0 + threadIdx.x);
        }
        if (threadIdx.x == 0) gstore(p.ws_ticket + r, 0u);  // self-restoring
        __syncthreads();
        uint32_t th = 0, tup = 0;
        bool lost = false;  // some list outgrew its slots
        for (int q = 0; q < eff; ++q) {
            th += sm.seg_hi[q];
            tup += sm.seg_lo[q] & 0x7FFFFFFFu;
            lost |= (sm.seg_lo[q] >> 31) != 0;
        }
        if (th < (uint32_t)p.k || lost || forced) {
            if (threadIdx.x == 0 && (th < (uint32_t)p.k || lost))
                gatomic_add(p.ws_stats + (lost ? 0 : 1), 1u);
            __syncthreads();
            select_and_emit<DT, Policy>(sm, p, r, base, row, RowSrc<DT, ORD>{row, (uint32_t)n});
            VTS_STAMP(4);
            return;
        }
        const bool rupper = tup >= (uint32_t)p.k;
        if (threadIdx.x == 0 && !rupper) gatomic_add(p.ws_stats + 3, 1u);
        select_and_emit<DT, Policy>(
            sm, p, r, base, row,
            MergeSrc{eff, rupper ? G.T2 : 0u, (uint32_t)p.ws_slots, p.ws_key + (size_t)unit0 * (uint32_t)p.ws_slots,
                     p.ws_idx + (size_t)unit0 * (uint32_t)p.ws_slots});
        VTS_STAMP(4);
        return;
    }
    const uint32_t lcap = refiltered ? (uint32_t)CAP : B.lds_cap;
    const uint32_t own = nh < lcap ? nh : lcap;
    // rank the keys >= T2 when at least k of them exist, else the whole list
    // (a re-filtered list has no T2 count: all of it)
    const bool whole_list = refiltered;
    const bool upper = !whole_list && nup >= (uint32_t)p.k;

    if (eff == 1 || direct) {  // one unit holds every candidate of the row
        if (nh < (uint32_t)p.k || p.force_path == FORCE_FALLBACK) {
            if (threadIdx.x == 0 && nh < (uint32_t)p.k) gatomic_add(p.ws_stats + 1, 1u);
            __syncthreads();
            whole_row<DT, Policy>(sm, p, r, base, n, row);
            VTS_STAMP(4);
            return;
        }
        if (threadIdx.x == 0 && !upper && !whole_list) gatomic_add(p.ws_stats + 3, 1u);
        const uint32_t thr = upper ? G.T2 : 0u;
        if (nh <= own) {  // every candidate on chip: the usual case
            select_and_emit<DT, Policy>(sm, p, r, base, row, LdsSrc<ONCHIP_J>(sm, nh, thr));
            VTS_STAMP(4);
            return;
        }
        if (nh <= (uint32_t)(20 * NT)) {
            // the on-chip slots and the spilled ones, selected as they are
            if (threadIdx.x == 0) gatomic_add(p.ws_stats + 2, 1u);
            select_and_emit<DT, Policy>(sm, p, r, base, row, LdsSrc<20>(sm, own, gkey, gidx, nh, thr));
            VTS_STAMP(4);
            return;
        }
        // a long spill: pull it into LDS with the compaction filter
        if (threadIdx.x == 0) {
            sm.cand_n = own;
            gatomic_add(p.ws_stats + 2, 1u);
        }
        __syncthreads();
        Thr<ORD> th = make_thr<ORD>(p, upper ? G.T2 : G.T);
        ingest_global<DT>(sm, p.k, gkey + own, gidx + own, nh - own, th);
        __syncthreads();
        const uint32_t m = sm.cand_n;
        __syncthreads();
        select_and_emit<DT, Policy>(sm, p, r, base, row, LdsSrc<ONCHIP_J>(sm, m));
        VTS_STAMP(4);
        return;
    }

    // split row: publish this unit's on-chip candidates, then take a ticket
    VTS_STAMP(11);
    for (uint32_t q = threadIdx.x; q < own; q += NT) {
        gstore(gkey + q, sm.key[q]);
        gstore(gidx + q, sm.idx[q]);
    }
    if (threadIdx.x == 0) {
        // a re-filtered unit's list holds its chunk's top k (or every key >=
        // T) with no T2 count: the flag makes the merge rank every list whole
        gstore(p.ws_count + unit, nh);
        gstore(p.ws_count_up + unit, nup | (whole_list ? 0x80000000u : 0u));
    }
    // Hand-off: the barrier orders every thread's candidate stores before
    // thread 0's agent-scope release fence, which precedes the ticket; the
    // unit that takes the last ticket issues an agent-scope acquire fence
    // before the barrier that releases its other threads to read.  One fence
    // per workgroup: each one writes back or invalidates the whole L2.
    __syncthreads();
    VTS_STAMP(12);
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const uint32_t old = __hip_atomic_fetch_add((VTS_GLOBAL uint32_t*)(p.ws_ticket + r), 1u,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = old == (uint32_t)eff - 1u;
        if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        sm.flag = last ? 1u : 0u;
    }
    __syncthreads();
    VTS_STAMP(5);
    if (sm.flag == 0) return;

    // last unit of the row: merge
    const uint32_t* rkey = p.ws_key + (size_t)unit0 * (uint32_t)p.ws_slots;
    const uint32_t* ridx = p.ws_idx + (size_t)unit0 * (uint32_t)p.ws_slots;
    // With at most GL lists, the first GL_SLOTS entries of every list (of
    // this unit's own list: its spilled entries from slot own on) are read
    // now, before their counts are known, so that the lists and the counts
    // arrive in one round trip; entries past a list's count are dropped
    // below.  Register e holds entry (e % GPL) * NT + thread of list e / GPL.
    // 32-bit keys only: measured on the 16-bit kernels (two lists per split
    // row there), the read-ahead cost more than the round trip it saves.
    constexpr int GL = 4, GPL = 4, GS = GL * GPL;
    constexpr int GLB = 8;  // lists whose bounds the gather below keeps in registers
    constexpr uint32_t GL_SLOTS = (uint32_t)(GPL * NT);
    static_assert(GL_SLOTS <= (uint32_t)HI_SLOTS, "read-ahead within a unit's workspace slots");
    const bool ahead = Traits<DT>::BITS > 16 && eff <= GL && (uint32_t)p.ws_slots >= own + GL_SLOTS;
    uint32_t gk[GS], gi[GS];
    if (ahead) {
#pragma unroll
        for (int e = 0; e < GS; ++e) {
            const int q = e / GPL;
            const uint32_t j = (uint32_t)(e % GPL) * NT + threadIdx.x + (q == c ? own : 0u);
            gk[e] = 0u;
            gi[e] = 0u;
            if (q < eff && (q != c || j < nh)) {
                gk[e] = gload(rkey + (size_t)q * (uint32_t)p.ws_slots + j);
                gi[e] = gload(ridx + (size_t)q * (uint32_t)p.ws_slots + j);
            }
        }
    }
    if (threadIdx.x < (unsigned)eff) {
        sm.seg_hi[threadIdx.x] = gload(p.ws_count + unit0 + threadIdx.x);
        sm.seg_lo[threadIdx.x] = gload(p.ws_count_up + unit0 + threadIdx.x);
    }
    if (threadIdx.x == 0) gstore(p.ws_ticket + r, 0u);  // self-restoring
    __syncthreads();
    VTS_STAMP(10);
    uint32_t th = 0, tup = 0;
    bool mixed = false;  // some unit was re-filtered
    for (int q = 0; q < eff; ++q) {
        th += sm.seg_hi[q];
        tup += sm.seg_lo[q] & 0x7FFFFFFFu;
        mixed |= (sm.seg_lo[q] >> 31) != 0;
    }
    if (th < (uint32_t)p.k || p.force_path == FORCE_FALLBACK) {
        if (threadIdx.x == 0 && th < (uint32_t)p.k) gatomic_add(p.ws_stats + 1, 1u);
        __syncthreads();
        whole_row<DT, Policy>(sm, p, r, base, n, row);
        VTS_STAMP(4);
        return;
    }
    const bool rupper = !mixed && tup >= (uint32_t)p.k;
    if (threadIdx.x == 0) {
        if (th > (uint32_t)CAP) gatomic_add(p.ws_stats + 2, 1u);
        if (!rupper) gatomic_add(p.ws_stats + 3, 1u);
    }
    if (th <= (uint32_t)CAP) {
        // Every list fits on chip: this unit's candidates stay in LDS slots
        // [0, own); the rest -- the other units' lists and this unit's spill,
        // m entries in all -- are gathered behind them in one pass, eight
        // entries per thread per round with all their loads in flight, and
        // the row is selected directly.  seg_lo now holds each list's first
        // gathered slot.
        const uint32_t m = th - own;
        // the read-ahead holds every list whole: place its entries behind
        // this unit's on-chip ones, list after list
        uint32_t gcount[GL], gbase[GL];
        bool whole = ahead;
        uint32_t acc = own;
#pragma unroll
        for (int q = 0; q < GL; ++q) {
            gcount[q] = 0u;
            if (q < eff) gcount[q] = sm.seg_hi[q] - (q == c ? own : 0u);
            gbase[q] = acc;
            acc += gcount[q];
            whole = whole && gcount[q] <= GL_SLOTS;
        }
        if (whole) {
#pragma unroll
            for (int e = 0; e < GS; ++e) {
                const int q = e / GPL;
                const uint32_t j = (uint32_t)(e % GPL) * NT + threadIdx.x;
                if (q < eff && j < gcount[q]) {
                    sm.key[gbase[q] + j] = gk[e];
                    sm.idx[gbase[q] + j] = gi[e];
                }
            }
            __syncthreads();
            select_and_emit<DT, Policy>(sm, p, r, base, row, LdsSrc<ONCHIP_J>(sm, th, rupper ? G.T2 : 0u));
            VTS_STAMP(4);
            return;
        }
        if (!ORD && !ahead && eff <= GLB) {  // (lists not read ahead; ORD: registers)
            // At most GLB lists: gathered entry i of list q (lists in order,
            // entry i at or past its first gathered slot gb[q]) is workspace
            // entry i + dl[q] from the row's first list; the list of each
            // entry is found by comparisons with the bounds, which every lane
            // holds (no loop over LDS), eight entries per thread per round
            // with all their loads in flight.
            uint32_t gb[GLB], dl[GLB];
            uint32_t acc = 0;
#pragma unroll
            for (int q = 0; q < GLB; ++q) {
                const uint32_t from = q == c ? own : 0u;
                gb[q] = q < eff ? acc : 0xFFFFFFFFu;
                dl[q] = (uint32_t)q * (uint32_t)p.ws_slots + from - acc;  // (mod 2^32)
                if (q < eff) acc += sm.seg_hi[q] - from;
            }
            constexpr int E = 8;
            for (uint32_t b0 = 0; b0 < m; b0 += (uint32_t)NT * E) {
                uint32_t kk[E], cc[E];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const uint32_t i = b0 + (uint32_t)e * NT + threadIdx.x;
                    uint32_t d = dl[0];
#pragma unroll
                    for (int q = 1; q < GLB; ++q) d = i >= gb[q] ? dl[q] : d;
                    const uint32_t at = i < m ? i + d : 0u;  // < (unit's lists) * ws_slots
                    kk[e] = gload(rkey + at);
                    cc[e] = gload(ridx + at);
                }
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const uint32_t i = b0 + (uint32_t)e * NT + threadIdx.x;
                    if (i < m) {
                        sm.key[own + i] = kk[e];
                        sm.idx[own + i] = cc[e];
                    }
                }
            }
            __syncthreads();
            select_and_emit<DT, Policy>(sm, p, r, base, row, LdsSrc<ONCHIP_J>(sm, th, rupper ? G.T2 : 0u));
            VTS_STAMP(4);
            return;
        }
        __syncthreads();  // every thread has read the counts in seg_lo
        if (threadIdx.x == 0) {
            uint32_t acc = 0;
            for (int q = 0; q < eff; ++q) {
                sm.seg_lo[q] = acc;
                acc += sm.seg_hi[q] - (q == c ? own : 0u);
            }
        }
        __syncthreads();
        constexpr int E = 8;
        for (uint32_t b0 = 0; b0 < m; b0 += (uint32_t)NT * E) {
            uint32_t kk[E], cc[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const uint32_t i = b0 + (uint32_t)e * NT + threadIdx.x;
                kk[e] = 0u;
                cc[e] = 0u;
                if (i < m) {
                    int q = 0;  // the list holding gathered entry i
                    while (q + 1 < eff && sm.seg_lo[q + 1] <= i) ++q;
                    const size_t at = (size_t)q * (uint32_t)p.ws_slots + (i - sm.seg_lo[q]) +
                                      (q == c ? own : 0u);
                    kk[e] = gload(rkey + at);
                    cc[e] = gload(ridx + at);
                }
            }
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const uint32_t i = b0 + (uint32_t)e * NT + threadIdx.x;
                if (i < m) {
                    sm.key[own + i] = kk[e];
                    sm.idx[own + i] = cc[e];
                }
            }
        }
        __syncthreads();
        select_and_emit<DT, Policy>(sm, p, r, base, row, LdsSrc<ONCHIP_J>(sm, th, rupper ? G.T2 : 0u));
        VTS_STAMP(4);
        return;
    }
    // Too many for the on-chip slots: this unit's candidates stay in place and
    // the others are pulled in with the compaction filter.
    if (threadIdx.x == 0) sm.cand_n = own;
    __syncthreads();
    Thr<ORD> thr = make_thr<ORD>(p, rupper ? G.T2 : G.T);
    for (int q = 0; q < eff; ++q) {
        const uint32_t mq = sm.seg_hi[q];
        const uint32_t from = q == c ? own : 0u;
        if (mq > from)
            ingest_global<DT>(sm, p.k, rkey + (size_t)q * (uint32_t)p.ws_slots + from,
                              ridx + (size_t)q * (uint32_t)p.ws_slots + from, mq - from, thr);
    }
    __syncthreads();
    const uint32_t m = sm.cand_n;
    __syncthreads();
    select_and_emit<DT, Policy>(sm, p, r, base, row, LdsSrc<ONCHIP_J>(sm, m, rupper ? G.T2 : 0u));
    VTS_STAMP(4);
}

template <int DT, class Policy, bool WIDE = false, bool HINT = false>
__global__ void __launch_bounds__(NT) topk_kernel(Params p) {
    __shared__ Smem sm;
    // units of one row are consecutive and land on one XCD (dispatch is
    // round-robin over the 8 XCDs by block index)
    const uint32_t bid = blockIdx.x;
    const uint32_t unit = (bid & 7u) * (uint32_t)p.units_per_xcd + (bid >> 3);
    if (unit >= (uint32_t)p.num_units) return;
    if constexpr (Policy::ORDERED) {
        if (threadIdx.x == 0) sm.sort_m = NO_SORT;
    }
    topk_unit<DT, Policy, WIDE, HINT>(sm, p, bid, unit);
    if constexpr (Policy::ORDERED) {
        lds_sync();
        const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)sm.sort_m);
        if (m != NO_SORT) {
            const int r = __builtin_amdgcn_readfirstlane((int)sm.sort_r);
            const int64_t base = __builtin_amdgcn_readfirstlane((int)sm.sort_base);
            const auto* row = static_cast<const typename Traits<DT>::raw_t*>(p.x) + (int64_t)r * p.row_stride + base;
            sort_and_emit<DT, Policy>(sm, p, r, base, row, m);
            VTS_STAMP(4);
        }
    }
}

}  // namespace vts
