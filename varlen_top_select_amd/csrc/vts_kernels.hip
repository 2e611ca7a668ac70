// vts_kernels.hip -- exact variable-length top-k selection for gfx950.
//
// One kernel serves a whole batch.  Each workgroup owns one (row, chunk) unit:
//
//  1. prologue: the row's valid window [base, base + n) is derived on the
//     device -- from seq_lens, next_n and compress_ratio (FlashInfer
//     top_k_varlen doc, `seq_lens`) or from lengths / row_starts (SGLang
//     TopK_Ops, fast_topk_v2).  n == 0 and n <= k rows are answered directly
//     (TensorRT-LLM PR #17821, short-row commit: identity then -1).
//  2. threshold: a fixed sample of the row (64 blocks of 64 contiguous
//     columns, or the whole row when it is short) is radix-selected in LDS at a
//     rank chosen so that, for exchangeable data, at least k row elements
//     clear the threshold except with negligible probability (the
//     sample-calibrated threshold of the self-sampling GVR V2 description on
//     the TensorRT-LLM PR #17821 page).  All workgroups of a row compute the
//     same threshold.
//  3. filter: one coalesced pass over the unit's columns with 16-byte loads;
//     keys >= threshold are appended to LDS with wave-aggregated tickets,
//     spilling to the workspace when LDS is full.  If even the workspace slots
//     run out, the unit is re-filtered with a compaction filter that keeps at
//     most k candidates at any time (exact for any input, slower).
//  4. verify: exactness needs at least k candidates over the row (then every
//     top-k element cleared the threshold).  Otherwise the row is re-selected
//     over all its columns with the compaction filter (never for
//     exchangeable data; exactness never rests on the sample).
//  5. select: the k-th largest candidate key K and the count g of keys > K,
//     by 8-bit radix select in LDS.
//  6. epilogue: all keys > K and k - g keys == K are written (ties are
//     interchangeable); indices are window-relative.  The page-table policy
//     applies the compact transform of the FlashInfer page-size PR body.
//
// Rows long enough get several workgroups (a split row).  Each writes its
// candidates to the workspace, then takes a ticket; the last one merges the
// candidates (steps 4-6) and resets the ticket, leaving the workspace clean.
// No workgroup ever waits for another.

#include "vts_device.hpp"
#include "vts_internal.h"

namespace vts {

// ---------------------------------------------------------------------------
// row windows and output policies
// ---------------------------------------------------------------------------

struct VarlenPolicy {
    // FlashInfer top_k_varlen doc, `seq_lens`: row t of request i ranks its
    // first max(0, (seq_lens[i] - next_n + t + 1) // compress_ratio) columns,
    // clamped to the width.
    __device__ __forceinline__ static void window(const Params& p, int r, int64_t& base, int64_t& n) {
        const int i = r / p.next_n, t = r - i * p.next_n;
        const int64_t num = (int64_t)gload(p.seq_lens + i) - p.next_n + t + 1;
        int64_t v = num <= 0 ? 0 : num / p.cr;
        n = v < p.width ? v : p.width;
        base = 0;
    }
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
};

struct PagePolicy {
    // Window [row_start, row_start + n), n = clamp(length, 0, width - row_start);
    // a start outside [0, width] is an empty row.
    __device__ __forceinline__ static void window(const Params& p, int r, int64_t& base, int64_t& n) {
        const int64_t b = p.row_starts ? (int64_t)gload(p.row_starts + r) : 0;
        const int64_t len = gload(p.lengths + r);
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
    __device__ __forceinline__ static int32_t translate(const Params& p, int r, int64_t base, int32_t col) {
        if (col < 0) return -1;
        const int64_t start = p.ptrs ? (int64_t)gload(p.ptrs + r) : base;
        const int64_t pc = start + col / p.page_size;
        if (pc < 0 || pc >= p.pt_width) return -1;
        const int64_t page = gload(p.pt + (int64_t)r * p.pt_stride + pc);
        return (int32_t)(page * p.page_size + col % p.page_size);
    }
    template <int DT>
    __device__ __forceinline__ static void emit(const Params& p, int r, int64_t base, uint32_t pos, int32_t col,
                                uint32_t) {
        const int64_t o = (int64_t)r * p.k + pos;
        gstore(p.out_idx + o, translate(p, r, base, col));
        if (p.out_raw) gstore(p.out_raw + o, col);
    }
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

// Keys of one streaming step held by a thread: U vectors of VE elements.
template <int DT>
struct StepRegs {
    static constexpr int VE = Traits<DT>::VE;
    static constexpr int KPT = U * VE;
    u32x4 v[U];
};

template <int DT>
__device__ __forceinline__ void load_step(StepRegs<DT>& R, const u32x4* vbase, int64_t v_begin,
                                          int64_t v_end) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t v = v_begin + (int64_t)u * NT + threadIdx.x;
        if (v < v_end) R.v[u] = gload(vbase + v);
    }
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
// logical candidate buffer: slots [0, lds_cap) in LDS, [lds_cap, gcap) in the
// unit's workspace region
// ---------------------------------------------------------------------------

struct Buf {
    uint32_t* gkey;
    uint32_t* gidx;
    uint32_t lds_cap;
    uint32_t gcap;
};

// every lane of the wave calls this together
__device__ __forceinline__ void buf_append(Smem& sm, const Buf& B, bool pass, uint32_t key,
                                           uint32_t col) {
    uint64_t m;
    const uint32_t pos = wave_ticket(&sm.cand_n, pass, m);
    if (pass) {
        if (pos < B.lds_cap) {
            sm.key[pos] = key;
            sm.idx[pos] = col;
        } else if (pos < B.gcap) {
            gstore(B.gkey + pos, key);
            gstore(B.gidx + pos, col);
        }
    }
}

// ---------------------------------------------------------------------------
// sampled threshold
// ---------------------------------------------------------------------------

// Key T such that every workgroup of the row keeps keys >= T.  Rows with at
// most SAMPLE columns are read whole and T is their exact k-th largest key.
// Longer rows read SAMPLE_BLOCKS blocks of SAMPLE_BLOCK columns spread evenly
// over [0, n); T is the sample's q-th largest key with
//   q = ceil(mu + sigma * sqrt(mu) + 4),  mu = k * SAMPLE / n,
// mu being the expected number of sampled keys above the row's k-th largest.
template <int DT>
__device__ __forceinline__ uint32_t sample_threshold(Smem& sm, const Params& p,
                                     const typename Traits<DT>::raw_t* row, int64_t n) {
    uint32_t keys[SPT];
    uint32_t vmask = 0;
    uint32_t q;
    if (n <= SAMPLE) {
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
            const int64_t pos = threadIdx.x + (int64_t)j * NT;
            keys[j] = 0;
            if (pos < n) {
                keys[j] = to_key<DT>(gload(row + pos));
                vmask |= 1u << j;
            }
        }
        q = (uint32_t)p.k;
    } else {
        const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
            const int64_t b = w + j * WAVES;
            const int64_t start = b * (n - SAMPLE_BLOCK) / (SAMPLE_BLOCKS - 1);
            keys[j] = to_key<DT>(gload(row + start + lane));
        }
        vmask = (SPT >= 32) ? 0xFFFFFFFFu : ((1u << SPT) - 1u);
        const float mu = (float)p.k * (float)SAMPLE / (float)n;
        const float qf = ceilf(mu + p.sigma * sqrtf(mu) + 4.0f);
        q = qf >= (float)SAMPLE ? (uint32_t)SAMPLE : (uint32_t)qf;
    }
    uint32_t T, gt;
    block_select<Traits<DT>::BITS>(
        sm,
        [&](auto f) {
#pragma unroll
            for (int j = 0; j < SPT; ++j)
                if ((vmask >> j) & 1u) f(keys[j]);
        },
        q, T, gt);
    return T;
}

// ---------------------------------------------------------------------------
// fast filter: one pass, no barriers inside the loop
// ---------------------------------------------------------------------------

template <int DT>
__device__ __forceinline__ void filter_step(Smem& sm, const Buf& B, const StepRegs<DT>& R,
                                            int64_t v_begin, int64_t v_end, int64_t h,
                                            uint32_t T) {
    constexpr int VE = Traits<DT>::VE;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t v = v_begin + (int64_t)u * NT + threadIdx.x;
        const bool ok = v < v_end;
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            const uint32_t key = to_key<DT>(vec_elem<DT>(R.v[u], e));
            buf_append(sm, B, ok && key >= T, key, (uint32_t)(h + v * VE + e));
        }
    }
}

// scalar columns [a, b) of the window (at most a few), every thread calls
template <int DT>
__device__ __forceinline__ void filter_scalars(Smem& sm, const Buf& B,
                                               const typename Traits<DT>::raw_t* row, int64_t a,
                                               int64_t b, uint32_t T) {
    for (int64_t base = a; base < b; base += NT) {
        const int64_t c = base + threadIdx.x;
        const bool ok = c < b;
        const uint32_t key = ok ? to_key<DT>(gload(row + c)) : 0u;
        buf_append(sm, B, ok && key >= T, key, (uint32_t)c);
    }
}

// ---------------------------------------------------------------------------
// compaction filter: exact for any input; keeps at most CAP candidates in LDS
// ---------------------------------------------------------------------------

struct Thr {
    uint32_t T;
    bool strict;  // pass: strict ? key > T : key >= T
    __device__ bool pass(uint32_t key) const { return strict ? key > T : key >= T; }
};

// Reduces LDS slots [0, cand_n) plus the calling threads' register keys that
// pass `thr` to exactly k entries: all keys > K and enough keys == K, where K
// is the k-th largest key of that union.  Afterwards only keys > K can matter.
template <int DT, int KPT>
__device__ __forceinline__ void compact(Smem& sm, int k, const uint32_t (&kk)[KPT], const uint32_t (&cc)[KPT],
                        uint32_t vm, Thr& thr, uint32_t old_n) {
    uint32_t K, gt;
    block_select<Traits<DT>::BITS>(
        sm,
        [&](auto f) {
            for (uint32_t q = threadIdx.x; q < old_n; q += NT) f(sm.key[q]);
#pragma unroll
            for (int j = 0; j < KPT; ++j)
                if (((vm >> j) & 1u) && thr.pass(kk[j])) f(kk[j]);
        },
        (uint32_t)k, K, gt);
    const uint32_t need_eq = (uint32_t)k - gt;
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
        const bool keep = (ok && key > K) || (iseq && e < need_eq);
        const uint32_t pos = wave_ticket(&sm.cnt_a, keep, m);
        if (keep) {
            sm.key[pos] = key;
            sm.idx[pos] = col;
        }
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const bool ok = ((vm >> j) & 1u) && thr.pass(kk[j]);
        uint64_t m;
        const bool iseq = ok && kk[j] == K;
        const uint32_t e = wave_ticket(&sm.cnt_b, iseq, m);
        const bool keep = (ok && kk[j] > K) || (iseq && e < need_eq);
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
    thr.strict = true;
}

// One compaction-filter step over register keys kk (valid mask vm).
template <int DT, int KPT>
__device__ __forceinline__ void careful_step(Smem& sm, int k, const uint32_t (&kk)[KPT],
                                             const uint32_t (&cc)[KPT], uint32_t vm, Thr& thr) {
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) cnt += (((vm >> j) & 1u) && thr.pass(kk[j])) ? 1u : 0u;
    uint32_t cand;
    const uint32_t total = block_sum(sm, cnt, cand);
    if (total == 0) return;
    if (cand + total > (uint32_t)CAP) {
        compact<DT, KPT>(sm, k, kk, cc, vm, thr, cand);
        return;
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const bool ok = ((vm >> j) & 1u) && thr.pass(kk[j]);
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
template <int DT>
__device__ __forceinline__ void careful_filter(Smem& sm, const Params& p, const typename Traits<DT>::raw_t* row,
                               const Slice& s, Thr thr) {
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
            kk[0] = vm ? to_key<DT>(gload(row + c)) : 0u;
            cc[0] = (uint32_t)c;
            careful_step<DT, 1>(sm, p.k, kk, cc, vm, thr);
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
            kk[e] = to_key<DT>(vec_elem<DT>(q, e));
            cc[e] = (uint32_t)(s.h + v * VE + e);
        }
        careful_step<DT, VE>(sm, p.k, kk, cc, vm, thr);
    }
}

// ---------------------------------------------------------------------------
// final selection and epilogue
// ---------------------------------------------------------------------------

// Enumerates candidate entries (key, col) with wave-uniform trip counts.
struct LdsSrc {
    uint32_t n;
    template <class F>
    __device__ __forceinline__ void for_each(Smem& sm, F f) const {
        for (uint32_t b = 0; b < n; b += NT) {
            const uint32_t q = b + threadIdx.x;
            const bool ok = q < n;
            f(ok, ok ? sm.key[q] : 0u, ok ? sm.idx[q] : 0u);
        }
    }
};

struct BufSrc {  // logical buffer: LDS slots [0, lds_n), workspace slots [lds_cap, n)
    uint32_t n, lds_cap;
    const uint32_t* gkey;
    const uint32_t* gidx;
    template <class F>
    __device__ __forceinline__ void for_each(Smem& sm, F f) const {
        const uint32_t nl = n < lds_cap ? n : lds_cap;
        for (uint32_t b = 0; b < nl; b += NT) {
            const uint32_t q = b + threadIdx.x;
            const bool ok = q < nl;
            f(ok, ok ? sm.key[q] : 0u, ok ? sm.idx[q] : 0u);
        }
        for (uint32_t b = lds_cap; b < n; b += NT) {
            const uint32_t q = b + threadIdx.x;
            const bool ok = q < n;
            f(ok, ok ? gload(gkey + q) : 0u, ok ? gload(gidx + q) : 0u);
        }
    }
};

struct SegSrc {  // the workspace regions of a split row's units
    int nseg;
    const uint32_t* gkey;  // region of unit 0 of the row
    const uint32_t* gidx;
    template <class F>
    __device__ __forceinline__ void for_each(Smem& sm, F f) const {
        for (int s = 0; s < nseg; ++s) {
            const uint32_t n = sm.seg_cnt[s];
            const uint32_t* kp = gkey + (size_t)s * WSCAP;
            const uint32_t* ip = gidx + (size_t)s * WSCAP;
            for (uint32_t b = 0; b < n; b += NT) {
                const uint32_t q = b + threadIdx.x;
                const bool ok = q < n;
                f(ok, ok ? gload(kp + q) : 0u, ok ? gload(ip + q) : 0u);
            }
        }
    }
};

// Selects the top k of `src` (which must hold at least k entries and contain
// a top-k of the row) and writes them through the policy.
template <int DT, class Policy, class Src>
__device__ __forceinline__ void select_and_emit(Smem& sm, const Params& p, int r, int64_t base, const Src& src) {
    uint32_t K, gt;
    block_select<Traits<DT>::BITS>(
        sm,
        [&](auto f) {
            src.for_each(sm, [&](bool ok, uint32_t key, uint32_t) {
                if (ok) f(key);
            });
        },
        (uint32_t)p.k, K, gt);
    const uint32_t need_eq = (uint32_t)p.k - gt;
    if (threadIdx.x == 0) {
        sm.cnt_a = 0;
        sm.cnt_b = 0;
    }
    __syncthreads();
    src.for_each(sm, [&](bool ok, uint32_t key, uint32_t col) {
        uint64_t m;
        const bool isgt = ok && key > K;
        const uint32_t pg = wave_ticket(&sm.cnt_a, isgt, m);
        if (isgt) Policy::template emit<DT>(p, r, base, pg, (int32_t)col, from_key<DT>(key));
        const bool iseq = ok && key == K;
        const uint32_t e = wave_ticket(&sm.cnt_b, iseq, m);
        if (iseq && e < need_eq)
            Policy::template emit<DT>(p, r, base, gt + e, (int32_t)col, from_key<DT>(key));
    });
}

template <int DT, class Policy>
__device__ __forceinline__ void short_row(const Params& p, int r, int64_t base, int64_t n,
                          const typename Traits<DT>::raw_t* row) {
    for (int j = threadIdx.x; j < p.k; j += NT) {
        const bool in = j < n;
        Policy::template emit<DT>(p, r, base, (uint32_t)j, in ? j : -1,
                                  in ? (uint32_t)gload(row + j) : Traits<DT>::PAD);
    }
}

// Whole-row re-selection with the compaction filter (threshold: everything).
template <int DT, class Policy>
__device__ __forceinline__ void whole_row(Smem& sm, const Params& p, int r, int64_t base, int64_t n,
                          const typename Traits<DT>::raw_t* row) {
    const Slice s = make_slice<DT>(row, n, 0, 1);
    careful_filter<DT>(sm, p, row, s, Thr{0u, false});
    __syncthreads();
    const uint32_t cand = sm.cand_n;
    __syncthreads();
    select_and_emit<DT, Policy>(sm, p, r, base, LdsSrc{cand});
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

template <int DT, class Policy>
__global__ void __launch_bounds__(NT) topk_kernel(Params p) {
    using raw_t = typename Traits<DT>::raw_t;
    __shared__ Smem sm;

    // units of one row are consecutive and land on one XCD (dispatch is
    // round-robin over the 8 XCDs by block index)
    const uint32_t bid = blockIdx.x;
    const uint32_t unit = (bid & 7u) * (uint32_t)p.units_per_xcd + (bid >> 3);
    if (unit >= (uint32_t)p.num_units) return;
    const int r = (int)(unit / (uint32_t)p.nsplit);
    const int c = (int)(unit - (uint32_t)r * (uint32_t)p.nsplit);

    int64_t base, n;
    Policy::window(p, r, base, n);
    const raw_t* row = static_cast<const raw_t*>(p.x) + (int64_t)r * p.row_stride + base;
    if (n <= p.k) {
        if (c == 0) short_row<DT, Policy>(p, r, base, n, row);
        return;
    }
    int64_t eff64 = (n + p.min_chunk - 1) / p.min_chunk;
    if (eff64 > p.nsplit) eff64 = p.nsplit;
    if (eff64 < 1) eff64 = 1;
    const int eff = (int)eff64;
    if (c >= eff) return;

    const Slice s = make_slice<DT>(row, n, c, eff);
    uint32_t* gkey = p.ws_key + (size_t)unit * WSCAP;
    uint32_t* gidx = p.ws_idx + (size_t)unit * WSCAP;
    const Buf B{gkey, gidx, (uint32_t)p.lds_cap, (uint32_t)p.wscap};
    const u32x4* vb = reinterpret_cast<const u32x4*>(row + s.h);
    const int64_t step = (int64_t)NT * U;

    // first streaming step is issued before the threshold is known
    StepRegs<DT> cur;
    if (p.force_path != FORCE_CAREFUL) load_step<DT>(cur, vb, s.v0, s.v1);
    if (threadIdx.x == 0) sm.cand_n = 0;
    const uint32_t T = sample_threshold<DT>(sm, p, row, n);

    bool in_lds_only = false;
    if (p.force_path != FORCE_CAREFUL) {
        filter_scalars<DT>(sm, B, row, s.s0, s.s1, T);
        for (int64_t vs = s.v0; vs < s.v1; vs += step) {
            StepRegs<DT> nxt;
            if (vs + step < s.v1) load_step<DT>(nxt, vb, vs + step, s.v1);
            filter_step<DT>(sm, B, cur, vs, s.v1, s.h, T);
            cur = nxt;
        }
        filter_scalars<DT>(sm, B, row, s.t0, s.t1, T);
        __syncthreads();
        const uint32_t filled = sm.cand_n;
        __syncthreads();  // everyone has read the count before it can change
        if (filled > B.gcap) {  // overflow: re-filter this unit with compaction
            if (threadIdx.x == 0) gatomic_add(p.ws_stats + 0, 1u);
            careful_filter<DT>(sm, p, row, s, Thr{T, false});
            in_lds_only = true;
        }
    } else {
        careful_filter<DT>(sm, p, row, s, Thr{T, false});
        in_lds_only = true;
    }
    __syncthreads();
    const uint32_t cand = sm.cand_n;
    __syncthreads();
    const uint32_t lcap = in_lds_only ? (uint32_t)CAP : B.lds_cap;

    if (eff == 1) {
        if (cand < (uint32_t)p.k || p.force_path == FORCE_FALLBACK) {
            if (threadIdx.x == 0 && cand < (uint32_t)p.k) gatomic_add(p.ws_stats + 1, 1u);
            __syncthreads();
            whole_row<DT, Policy>(sm, p, r, base, n, row);
            return;
        }
        select_and_emit<DT, Policy>(sm, p, r, base, BufSrc{cand, lcap, gkey, gidx});
        return;
    }

    // split row: publish this unit's candidates, then take a ticket
    {
        const uint32_t nl = cand < lcap ? cand : lcap;
        for (uint32_t q = threadIdx.x; q < nl; q += NT) {
            gstore(gkey + q, sm.key[q]);
            gstore(gidx + q, sm.idx[q]);
        }
        if (threadIdx.x == 0) gstore(p.ws_count + unit, cand);
    }
    // release: every thread's candidate stores, then the ticket (agent scope)
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        const uint32_t old = __hip_atomic_fetch_add((VTS_GLOBAL uint32_t*)(p.ws_ticket + r), 1u, __ATOMIC_ACQ_REL,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        sm.flag = (old == (uint32_t)eff - 1u) ? 1u : 0u;
        __threadfence();
    }
    __syncthreads();
    if (sm.flag == 0) return;
    __threadfence();  // acquire side for every thread of the merging workgroup

    // last unit of the row: merge
    const uint32_t unit0 = (uint32_t)r * (uint32_t)p.nsplit;
    if (threadIdx.x < (unsigned)eff) sm.seg_cnt[threadIdx.x] = gload(p.ws_count + unit0 + threadIdx.x);
    if (threadIdx.x == 0) gstore(p.ws_ticket + r, 0u);  // self-restoring
    __syncthreads();
    uint32_t total = 0;
    for (int q = 0; q < eff; ++q) total += sm.seg_cnt[q];
    const uint32_t* rkey = p.ws_key + (size_t)unit0 * WSCAP;
    const uint32_t* ridx = p.ws_idx + (size_t)unit0 * WSCAP;
    if (total < (uint32_t)p.k || p.force_path == FORCE_FALLBACK) {
        if (threadIdx.x == 0 && total < (uint32_t)p.k) gatomic_add(p.ws_stats + 1, 1u);
        __syncthreads();
        whole_row<DT, Policy>(sm, p, r, base, n, row);
        return;
    }
    if (total <= (uint32_t)p.lds_cap) {
        uint32_t off = 0;
        for (int q = 0; q < eff; ++q) {
            const uint32_t m = sm.seg_cnt[q];
            for (uint32_t i = threadIdx.x; i < m; i += NT) {
                sm.key[off + i] = gload(rkey + (size_t)q * WSCAP + i);
                sm.idx[off + i] = gload(ridx + (size_t)q * WSCAP + i);
            }
            off += m;
        }
        __syncthreads();
        select_and_emit<DT, Policy>(sm, p, r, base, LdsSrc{total});
    } else {
        if (threadIdx.x == 0) gatomic_add(p.ws_stats + 2, 1u);
        select_and_emit<DT, Policy>(sm, p, r, base, SegSrc{eff, rkey, ridx});
    }
}

// ---------------------------------------------------------------------------
// launches
// ---------------------------------------------------------------------------

template <int DT, class Policy>
static hipError_t launch_dt(const Params& p, hipStream_t stream) {
    const uint32_t grid = (uint32_t)p.units_per_xcd * 8u;
    hipLaunchKernelGGL((topk_kernel<DT, Policy>), dim3(grid), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_varlen(int dtype, const Params& p, hipStream_t stream) {
    switch (dtype) {
        case F32: return launch_dt<F32, VarlenPolicy>(p, stream);
        case BF16: return launch_dt<BF16, VarlenPolicy>(p, stream);
        case F16: return launch_dt<F16, VarlenPolicy>(p, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_transform(int dtype, const Params& p, hipStream_t stream) {
    switch (dtype) {
        case F32: return launch_dt<F32, PagePolicy>(p, stream);
        case BF16: return launch_dt<BF16, PagePolicy>(p, stream);
        case F16: return launch_dt<F16, PagePolicy>(p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace vts
