// vts_device.hpp -- device building blocks for the top-k kernels (gfx950, wave64).
//
//  * order-preserving unsigned keys for fp32 / bf16 / fp16;
//  * wave64 ballot / mbcnt helpers and wave-aggregated LDS counters;
//  * a workgroup radix select (10-bit digits from the first bit in which the
//    keys differ, a padded 1024-bin LDS histogram scanned by one wave) that
//    finds the exact r-th largest key of any key set that the workgroup can
//    enumerate, and a paired variant that finds two ranks at once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vts {

constexpr int NT = 256;               // threads per workgroup: 4 wave64
constexpr int WAVES = NT / 64;
constexpr int CAP = 3776;             // on-chip candidate slots per workgroup
constexpr int STAGE = 128;            // staged 16-byte vectors per wave
constexpr int STAGE_DRAIN = 64;       // a wave drains one full round at this many
constexpr int SAMPLE = 8192;          // sampled keys per row: 128 blocks of 64 columns
constexpr int SAMPLE_BLOCK = 64;      // columns per sample block
constexpr int SAMPLE_BLOCKS = SAMPLE / SAMPLE_BLOCK;
constexpr int SPT = SAMPLE / NT;      // sampled keys per thread (32)
static_assert(SPT <= 32, "one mask bit per sampled key of a thread");
constexpr int MAX_SPLIT = 32;         // workgroups per row, at most

enum Dtype : int { F32 = 0, BF16 = 1, F16 = 2 };

// Global-memory accesses through address-space-1 pointers, so the compiler
// emits global_* instructions.  Generic (flat) accesses would also count on
// the LDS wait counter, and every LDS ticket would then wait for all loads in
// flight.
#define VTS_GLOBAL __attribute__((address_space(1)))

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <class T>
__device__ __forceinline__ T gload(const T* p) {
    return *(const VTS_GLOBAL T*)p;
}
template <class T>
__device__ __forceinline__ void gstore(T* p, T v) {
    *(VTS_GLOBAL T*)p = v;
}
// p[i] = v with a 32-bit byte offset from the (wave-uniform) base, which lets
// the store take the scalar-base + 32-bit vector-offset address form
__device__ __forceinline__ void gstore_at(uint32_t* p, uint32_t i, uint32_t v) {
    *(VTS_GLOBAL uint32_t*)((VTS_GLOBAL char*)p + (i << 2)) = v;
}
__device__ __forceinline__ uint32_t gatomic_add(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add((VTS_GLOBAL uint32_t*)p, v, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
}

// U: 16-byte vectors per thread per streaming step.  Two steps are in
// registers at once (one being filtered, one in flight), and the filter keeps
// a pass mask per step, so U is sized to stay under 128 VGPRs (4 waves/SIMD).
template <int DT> struct Traits;
// KEY_PINF / KEY_NINF: the keys of +inf and -inf (see to_key); keys above
// KEY_PINF are NaNs with the sign clear, keys below KEY_NINF NaNs with it set.
template <> struct Traits<F32> {
    using raw_t = uint32_t;
    static constexpr int BITS = 32;
    static constexpr int VE = 4;  // elements per 16-byte vector
    static constexpr int U = 6;
    static constexpr uint32_t PAD = 0xFF7FFFFFu;  // -FLT_MAX
    static constexpr uint32_t KEY_PINF = 0xFF800000u, KEY_NINF = 0x007FFFFFu;
};
template <> struct Traits<BF16> {
    using raw_t = uint16_t;
    static constexpr int BITS = 16;
    static constexpr int VE = 8;
    static constexpr int U = 4;
    static constexpr uint32_t PAD = 0xFF7Fu;  // lowest finite bf16
    static constexpr uint32_t KEY_PINF = 0xFF80u, KEY_NINF = 0x007Fu;
};
template <> struct Traits<F16> {
    using raw_t = uint16_t;
    static constexpr int BITS = 16;
    static constexpr int VE = 8;
    static constexpr int U = 4;
    static constexpr uint32_t PAD = 0xFBFFu;  // lowest finite fp16
    static constexpr uint32_t KEY_PINF = 0xFC00u, KEY_NINF = 0x03FFu;
};

// Sign-magnitude float bits -> unsigned key whose integer order is the float
// order: negative values have all bits flipped, non-negative ones get the sign
// bit set.  -0 maps just below +0; NaNs land above +inf or below -inf.
template <int DT>
__device__ __forceinline__ uint32_t to_key(uint32_t raw) {
    if constexpr (Traits<DT>::BITS == 32) {
        return raw ^ ((uint32_t)((int32_t)raw >> 31) | 0x80000000u);
    } else {
        return (raw & 0x8000u) ? (~raw & 0xFFFFu) : (raw | 0x8000u);
    }
}

template <int DT>
__device__ __forceinline__ uint32_t from_key(uint32_t key) {
    if constexpr (Traits<DT>::BITS == 32) {
        return (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
    } else {
        return (key & 0x8000u) ? (key & 0x7FFFu) : (~key & 0xFFFFu);
    }
}

// Keys of the deterministic mode, where elements that compare as equal values
// must share one key: -0 takes the key of +0, every NaN with the sign clear
// the largest key and every NaN with the sign set the smallest.  The key
// order is then the value order (NaNs above +inf or below -inf) with every tie
// explicit, so a column tie-break makes it total.  Keys stay in the dtype's
// range; a canonical key no longer names its element's bits for -0 and NaN
// (canon_special), which are read back from the row where values are output.
template <int DT>
__device__ __forceinline__ uint32_t canon_key(uint32_t key) {
    constexpr uint32_t POS0 = Traits<DT>::BITS == 32 ? 0x80000000u : 0x8000u;
    constexpr uint32_t KMAX = Traits<DT>::BITS == 32 ? 0xFFFFFFFFu : 0xFFFFu;
    key = key == POS0 - 1u ? POS0 : key;
    key = key > Traits<DT>::KEY_PINF ? KMAX : key;
    return key < Traits<DT>::KEY_NINF ? 0u : key;
}

// whether a canonical key may stand for elements of other bits (+-0, NaN)
template <int DT>
__device__ __forceinline__ bool canon_special(uint32_t key) {
    constexpr uint32_t POS0 = Traits<DT>::BITS == 32 ? 0x80000000u : 0x8000u;
    constexpr uint32_t KMAX = Traits<DT>::BITS == 32 ? 0xFFFFFFFFu : 0xFFFFu;
    return key == POS0 || key == KMAX || key == 0u;
}

// The largest threshold t' <= t for which "canonical key >= t'" and the
// raw-bit test of RungTest (signed compare of the element bits with t's
// bits, used when t has the sign bit of a key set) agree on every element:
// +0's key becomes -0's (no canonical key equals it, and it is below +0, so
// the raw-bit test is not used), and a threshold inside the NaN range becomes
// the smallest NaN key (every NaN with the sign clear passes both tests).
// Lowering a threshold only admits more candidates.
template <int DT>
__device__ __forceinline__ uint32_t canon_floor(uint32_t t) {
    constexpr uint32_t POS0 = Traits<DT>::BITS == 32 ? 0x80000000u : 0x8000u;
    t = t > Traits<DT>::KEY_PINF + 1u ? Traits<DT>::KEY_PINF + 1u : t;
    return t == POS0 ? POS0 - 1u : t;
}

__device__ __forceinline__ uint32_t lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// number of set bits of m below this lane
__device__ __forceinline__ uint32_t mbcnt(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint32_t first_lane_value(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// Wave-aggregated ticket: every lane of the wave must call this together.
// Lanes with `want` receive consecutive tickets from *counter (LDS); the
// return value is meaningful only for them.
__device__ __forceinline__ uint32_t wave_ticket(uint32_t* counter, bool want, uint64_t& mask) {
    mask = ballot(want);
    if (mask == 0) return 0;
    uint32_t base = 0;
    if (lane_id() == 0) base = atomicAdd(counter, (uint32_t)__popcll(mask));
    base = first_lane_value(base);
    return base + mbcnt(mask);
}

constexpr int RBITS = 10;              // radix digit width of the selection
constexpr int NBINS = 1 << RBITS;      // 1024 histogram bins
// Bin d lives at LDS word d + d/16: one pad word per 16 bins, so the 64 lanes
// of the scanning wave, each reading 16 consecutive bins, hit distinct banks.
constexpr int HIST_WORDS = NBINS + NBINS / 16;
__device__ __forceinline__ uint32_t hslot(uint32_t d) { return d + (d >> 4); }

// Wave-aggregated ticket for variable counts: each lane asks for `cnt` (<= 127)
// consecutive slots of *counter (LDS); returns the lane's first slot.  The
// exclusive prefix of the counts is built from bit slices (one ballot and one
// mbcnt per bit), so only one LDS atomic is issued per wave.  Every lane of the
// wave must call it.
__device__ __forceinline__ uint32_t wave_ticket_n(uint32_t* counter, uint32_t cnt) {
    if (ballot(cnt != 0) == 0) return 0;
    uint32_t excl = 0, tot = 0;
#pragma unroll
    for (int b = 0; b < 7; ++b) {
        const uint64_t m = ballot((cnt >> b) & 1u);
        excl += mbcnt(m) << b;
        tot += (uint32_t)__popcll(m) << b;
    }
    uint32_t base = 0;
    if (lane_id() == 0) base = atomicAdd(counter, tot);
    return first_lane_value(base) + excl;
}

// wave_ticket_n for counts of any size (the wide selections enumerate
// hundreds of entries per thread): the exclusive prefix comes from a DPP scan
// of the wave.  Every lane of the wave must call it.
__device__ __forceinline__ uint32_t wave_ticket_any(uint32_t* counter, uint32_t cnt);

// Shared state of one workgroup (at most 40 KB, so four fit on a CU).  The
// selection histogram and the streaming filter's per-wave staging queues share
// their space: the queues exist only between two selections, and the
// histogram is cleared again after them.
struct Smem {
    union {
        struct {
            uint32_t key[CAP];
            uint32_t idx[CAP];
        };
        uint32_t cand_words[2 * CAP];  // both arrays, before any candidate exists
    };
    union {
        uint32_t hist[HIST_WORDS];
        struct {
            u32x4 vec[WAVES * STAGE];  // wave w owns [w * STAGE, (w + 1) * STAGE)
            uint32_t v[WAVES * STAGE];  // the vectors' indices in the unit's body
        } stage;
        // after the last selection: the page-table entries of the row's window
        uint32_t table[WAVES * STAGE * 5];
    };
    uint32_t wsum[WAVES];
    uint32_t wmin[WAVES];
    uint32_t wmax[WAVES];
    uint32_t seg_hi[MAX_SPLIT];
    uint32_t seg_lo[MAX_SPLIT];
    uint32_t cand_n;  // candidates: keys >= the safe rung (or compaction-filter entries)
    uint32_t up_n;    // of which keys >= the likely rung
    uint32_t cnt_a, cnt_b;
    uint32_t sel_digit, sel_above;
    uint32_t sel_digit2, sel_above2;
    uint32_t flag;
    uint32_t total;
    uint32_t win_base, win_n;  // the placed row's window (balanced placement)
    uint32_t sort_m, sort_r, sort_base;  // deterministic mode: the sort left to the kernel's end
    uint32_t row_n;  // the unit's row: valid columns of its window
#ifdef VTS_PHASE_STAMPS
    uint32_t stamp_unit;  // phase-timing build: the unit whose stamps this workgroup writes
#endif
};

constexpr int TABLE_WORDS = WAVES * STAGE * 5;
static_assert(sizeof(((Smem*)nullptr)->table) == sizeof(((Smem*)nullptr)->stage), "the table fills the staging area");

// Inclusive scan across the 64 lanes of a wave with DPP: Hillis-Steele inside
// each 16-lane row (row_shr 1, 2, 4, 8), then row_bcast 15 and 31 carry the
// row totals forward.  Lanes without a source get `identity`.
template <class Op>
__device__ __forceinline__ uint32_t wave_scan(uint32_t v, uint32_t identity, Op op) {
    const int id = (int)identity;
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x111, 0xF, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x112, 0xF, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x114, 0xF, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x118, 0xF, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x142, 0xA, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x143, 0xC, 0xF, false));
    return v;
}

// Workgroup barrier that orders LDS accesses only: the wave's own LDS
// operations complete (lgkmcnt), then s_barrier; the memory clobber keeps the
// compiler from moving memory accesses across it.  A full __syncthreads (and
// even an LDS-scoped fence) also waits for every global load still in flight,
// asynchronous loads into LDS included; this one lets them stay in flight, so
// it must not be used to publish LDS written by such loads (wait for them
// first) nor global memory written by other threads (use __syncthreads).
__device__ __forceinline__ void lds_sync() {
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

struct OpAdd { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };
struct OpMin { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; } };
struct OpMax { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; } };

__device__ __forceinline__ uint32_t wave_ticket_any(uint32_t* counter, uint32_t cnt) {
    const uint32_t incl = wave_scan(cnt, 0u, OpAdd());
    const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    if (tot == 0) return 0;  // uniform
    uint32_t base = 0;
    if (lane_id() == 0) base = atomicAdd(counter, tot);
    return first_lane_value(base) + incl - cnt;
}

// Inclusive prefix sum over the workgroup (thread order).  Contains barriers
// (LDS-only, as in every helper below): every thread must call it.
__device__ __forceinline__ uint32_t block_inclusive_scan(Smem& sm, uint32_t v) {
    v = wave_scan(v, 0u, OpAdd());
    const uint32_t w = threadIdx.x >> 6;
    if (lane_id() == 63) sm.wsum[w] = v;
    lds_sync();
    uint32_t add = 0;
#pragma unroll
    for (int i = 0; i < WAVES; ++i)
        if ((uint32_t)i < w) add += sm.wsum[i];
    lds_sync();
    return v + add;
}

// Workgroup sum of v.  Also returns, in cand_snapshot, the value of sm.cand_n
// read while no thread can change it (between the two barriers), so every
// thread takes the same decision on it.
__device__ __forceinline__ uint32_t block_sum(Smem& sm, uint32_t v, uint32_t& cand_snapshot) {
    uint32_t incl = block_inclusive_scan(sm, v);
    if (threadIdx.x == NT - 1) sm.total = incl;
    lds_sync();
    const uint32_t t = sm.total;
    cand_snapshot = sm.cand_n;
    lds_sync();
    return t;
}

// Workgroup-wide min and max (every thread must call; one barrier).  The
// per-wave slots are rewritten only by the next call, which is separated from
// this one by other barriers.
__device__ __forceinline__ void block_minmax(Smem& sm, uint32_t& lo, uint32_t& hi) {
    lo = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan(lo, 0xFFFFFFFFu, OpMin()), 63);
    hi = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan(hi, 0u, OpMax()), 63);
    const uint32_t w = threadIdx.x >> 6;
    if (lane_id() == 0) {
        sm.wmin[w] = lo;
        sm.wmax[w] = hi;
    }
    lds_sync();
    lo = sm.wmin[0];
    hi = sm.wmax[0];
#pragma unroll
    for (int i = 1; i < WAVES; ++i) {
        lo = sm.wmin[i] < lo ? sm.wmin[i] : lo;
        hi = sm.wmax[i] > hi ? sm.wmax[i] : hi;
    }
}

// Copies of the first-pass histogram of block_select_pair, in the candidate
// arrays (free until candidates arrive); the stride shifts each copy by one
// LDS bank.
constexpr int SPREAD_COPIES = 4;
constexpr int SPREAD_STRIDE = NBINS + 1;
static_assert(SPREAD_COPIES * SPREAD_STRIDE <= 2 * CAP, "copies fit in the candidate arrays");

__device__ __forceinline__ void spread_clear(Smem& sm) {
    for (int j = threadIdx.x; j < SPREAD_COPIES * SPREAD_STRIDE; j += NT) sm.cand_words[j] = 0;
}

// Zeroes the selection histogram; every select leaves it zeroed again.
__device__ __forceinline__ void hist_clear(Smem& sm) {
    // unrolled: no loop for the compiler's wait counts to merge over
#pragma unroll
    for (int i = 0; i < (HIST_WORDS + NT - 1) / NT; ++i) {
        const int j = (int)threadIdx.x + i * NT;
        if (j < HIST_WORDS) sm.hist[j] = 0;
    }
}

// Run by the 64 lanes of one wave after a barrier: bins [base, base + 64*PER)
// hold digit counts (digit d at bin base + d).  For each of the ranks r1 and
// r2 (1-based, counted from the largest digit; each at most the total) finds
// the digit holding that rank and the count of the digits above it, then
// zeroes the bins.  Lane l sums digits 64*PER-1-PER*l down to 64*PER-PER*(l+1);
// a DPP scan and a ballot name the lane where the count crosses r, then PER
// lanes read that lane's bins once more and a second scan names the digit.
// b1 receives the count of digit d1 itself.
template <int PER>
__device__ __forceinline__ void hist_crossing(Smem& sm, uint32_t base, uint32_t r1, uint32_t r2,
                                              uint32_t& d1, uint32_t& a1, uint32_t& d2,
                                              uint32_t& a2, uint32_t& b1) {
    constexpr uint32_t NB = 64u * PER;
    const uint32_t l = lane_id();
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) sum += sm.hist[hslot(base + NB - 1 - (l * PER + j))];
    const uint32_t incl = wave_scan(sum, 0u, OpAdd());
    const uint32_t excl = incl - sum;
    uint32_t b2;
    auto find = [&](uint32_t r, uint32_t& d, uint32_t& a, uint32_t& b) {
        const uint64_t m = ballot(incl >= r);
        const int L = m ? __builtin_ctzll(m) : 63;
        const uint32_t exL = (uint32_t)__builtin_amdgcn_readlane((int)excl, L);
        const uint32_t c = l < (uint32_t)PER ? sm.hist[hslot(base + NB - 1 - ((uint32_t)L * PER + l))] : 0u;
        const uint32_t ic = wave_scan(c, 0u, OpAdd());
        const uint64_t m2 = ballot(l < (uint32_t)PER && exL + ic >= r);
        const int J = m2 ? __builtin_ctzll(m2) : PER - 1;
        d = NB - 1 - ((uint32_t)L * PER + (uint32_t)J);
        a = exL + (uint32_t)__builtin_amdgcn_readlane((int)(ic - c), J);
        b = (uint32_t)__builtin_amdgcn_readlane((int)c, J);
    };
    find(r1, d1, a1, b1);
    if (r2 == r1) {
        d2 = d1;
        a2 = a1;
    } else {
        find(r2, d2, a2, b2);
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) sm.hist[hslot(base + NB - 1 - (l * PER + j))] = 0;
}

// Radix select over the key set that `visit` enumerates: visit(f) must call
// f(key) once for every key this thread owns (any order, any divergence).
// Finds the r-th largest key (1-based; the set must hold at least r keys),
// resolving its bits from the highest one in which lo and hi differ down to
// bit `min_bit`, 10 bits per pass.  Keys whose bits above that one differ
// from lo's are not counted, so every key must share them (lo <= every key
// <= hi guarantees it).  Returns in kth the key's bits >= min_bit (lower bits
// zero), so kth is a lower bound of the r-th largest key, and exact when
// min_bit == 0; n_greater counts the keys whose bits >= min_bit exceed kth's
// (with min_bit == 0: the keys strictly greater than the r-th largest, so
// r - n_greater keys equal to it complete the top r).
// Each pass: every thread adds its matching keys' digits into 1024 LDS bins;
// after a barrier wave 0 alone finds the digit holding the remaining rank and
// zeroes the bins; a second barrier publishes the digit.  The histogram must
// be zero on entry and is zero on exit.  Every thread must call it.
// RANGE: the passes may also end early, once the digit holding the remaining
// rank holds exactly that many keys: every key of it then belongs to the top
// r, whatever its unresolved low bits.  kth_top receives the largest key the
// resolved digits allow (kth with every unresolved bit set), so the top r is
// the n_greater keys above kth_top and the r - n_greater keys in
// [kth, kth_top]; without an early end, kth_top = kth | (bits below min_bit).
template <bool RANGE, class Visit>
__device__ __forceinline__ void block_select_bits(Smem& sm, Visit visit, uint32_t r, uint32_t lo,
                                                  uint32_t hi, int min_bit, uint32_t& kth,
                                                  uint32_t& kth_top, uint32_t& n_greater) {
    const uint32_t low_mask = min_bit >= 32 ? 0xFFFFFFFFu : ((1u << min_bit) - 1u);
    if (((lo ^ hi) & ~low_mask) == 0) {  // all keys share the bits that matter
        kth = lo & ~low_mask;
        kth_top = kth | low_mask;
        n_greater = 0;
        // (uniform branch) the barrier that a pass would end with: lo and hi
        // came from block_minmax, whose per-wave slots the next one rewrites
        lds_sync();
        return;
    }
    const int hb = 31 - __clz(lo ^ hi);
    uint32_t mask = hb == 31 ? 0u : ~((2u << hb) - 1u);
    uint32_t prefix = lo & mask;
    uint32_t krem = r, gt = 0;
    for (int top = hb; top >= min_bit; top -= RBITS) {
        int width = top + 1 - min_bit;
        if (width > RBITS) width = RBITS;
        const int shift = top + 1 - width;
        const uint32_t dmask = (1u << width) - 1u;
        visit([&](uint32_t key) {
            if ((key & mask) == prefix) atomicAdd(&sm.hist[hslot((key >> shift) & dmask)], 1u);
        });
        lds_sync();
        if (threadIdx.x < 64) {
            uint32_t d, a, d2, a2, b;
            hist_crossing<NBINS / 64>(sm, 0u, krem, krem, d, a, d2, a2, b);
            if (threadIdx.x == 0) {
                sm.sel_digit = d;
                sm.sel_above = a;
                sm.sel_digit2 = b;  // (a free word here) the digit's own count
            }
        }
        lds_sync();
        const uint32_t d = sm.sel_digit, above = sm.sel_above;
        gt += above;
        krem -= above;
        prefix |= d << shift;
        mask |= dmask << shift;
        if constexpr (RANGE) {
            if (sm.sel_digit2 == krem) break;  // (uniform) the whole digit completes the rank
        }
    }
    kth = prefix;
    kth_top = prefix | ~mask;
    n_greater = gt;
}

template <class Visit>
__device__ __forceinline__ void block_select(Smem& sm, Visit visit, uint32_t r, uint32_t lo,
                                             uint32_t hi, int min_bit, uint32_t& kth,
                                             uint32_t& n_greater) {
    uint32_t top;
    block_select_bits<false>(sm, visit, r, lo, hi, min_bit, kth, top, n_greater);
}

// Two lower bounds at once: the r1-th and r2-th largest keys of the set that
// `visit` enumerates (r1 >= r2, each at most the set's size), resolved to
// their top BITS - 10 + W2 bits.  Pass 1 takes the top 10 bits as the digit
// (1024 bins) and finds both ranks' digits; pass 2 takes the next W2 bits (at
// most 9) of the keys in each of those digits, in two 512-bin halves (one if
// both digits agree).  Histogram zero on entry and exit; every thread calls.
template <int BITS, int W2, class Visit>
__device__ __forceinline__ void block_select_pair(Smem& sm, Visit visit, uint32_t r1, uint32_t r2,
                                                  uint32_t& k1, uint32_t& k2) {
    static_assert(W2 >= 1 && W2 <= 9 && BITS - RBITS - W2 >= 0, "digit widths");
    constexpr int S1 = BITS - RBITS, S2 = S1 - W2;
    constexpr uint32_t M2 = (1u << W2) - 1u;
    // Pass 1 counts into SPREAD_COPIES copies of the histogram (lane l into
    // copy l % SPREAD_COPIES), which the candidate arrays hold before any
    // candidate exists: the top 10 bits of typical keys fall into a few digits,
    // and one copy would serialize many lanes of an atomic on one address.
    // The copies are then summed into the histogram (spread_clear zeroed them).
    uint32_t* spread = sm.cand_words;
    const uint32_t copy = (lane_id() % SPREAD_COPIES) * SPREAD_STRIDE;
    visit([&](uint32_t key) { atomicAdd(&spread[copy + (key >> S1)], 1u); });
    lds_sync();
    for (int b = threadIdx.x; b < NBINS; b += NT) {
        uint32_t t = 0;
#pragma unroll
        for (int c = 0; c < SPREAD_COPIES; ++c) t += spread[c * SPREAD_STRIDE + b];
        sm.hist[hslot(b)] = t;
    }
    lds_sync();
    if (threadIdx.x < 64) {
        uint32_t d1, a1, d2, a2;
        uint32_t b1;
        hist_crossing<NBINS / 64>(sm, 0u, r1, r2, d1, a1, d2, a2, b1);
        if (threadIdx.x == 0) {
            sm.sel_digit = d1;
            sm.sel_above = a1;
            sm.sel_digit2 = d2;
            sm.sel_above2 = a2;
        }
    }
    lds_sync();
    const uint32_t d1 = sm.sel_digit, d2 = sm.sel_digit2;
    const uint32_t q1 = r1 - sm.sel_above, q2 = r2 - sm.sel_above2;
    const uint32_t base2 = d2 == d1 ? 0u : 512u;
    visit([&](uint32_t key) {
        const uint32_t d = key >> S1, e = (key >> S2) & M2;
        if (d == d1) atomicAdd(&sm.hist[hslot(e)], 1u);
        if (d == d2 && base2) atomicAdd(&sm.hist[hslot(base2 + e)], 1u);
    });
    lds_sync();
    if (threadIdx.x < 64) {
        constexpr int PER = (1 << W2) / 64 > 0 ? (1 << W2) / 64 : 1;
        // with W2 < 6 the 64-lane view covers 64 bins; the digits above 2^W2 are zero
        uint32_t e1, b1, e2, b2, x, y, z;
        hist_crossing<PER>(sm, 0u, q1, base2 ? q1 : q2, e1, b1, x, y, z);
        if (base2) {
            hist_crossing<PER>(sm, base2, q2, q2, e2, b2, x, y, z);
        } else {
            e2 = x;
        }
        if (threadIdx.x == 0) {
            sm.sel_digit = (d1 << S1) | (e1 << S2);
            sm.sel_digit2 = (d2 << S1) | (e2 << S2);
        }
    }
    lds_sync();
    k1 = sm.sel_digit;
    k2 = sm.sel_digit2;
}

// Exact selection with the key range found first (one extra visit).
template <class Visit>
__device__ __forceinline__ void block_select_exact(Smem& sm, Visit visit, uint32_t r,
                                                   uint32_t& kth, uint32_t& n_greater) {
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    visit([&](uint32_t key) {
        lo = key < lo ? key : lo;
        hi = key > hi ? key : hi;
    });
    block_minmax(sm, lo, hi);
    block_select(sm, visit, r, lo, hi, 0, kth, n_greater);
}

// The same, allowed to end early: the top r are the n_greater keys above
// kth_top and the r - n_greater keys in [kth, kth_top] (block_select_bits).
template <class Visit>
__device__ __forceinline__ void block_select_range(Smem& sm, Visit visit, uint32_t r,
                                                   uint32_t& kth, uint32_t& kth_top,
                                                   uint32_t& n_greater) {
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    visit([&](uint32_t key) {
        lo = key < lo ? key : lo;
        hi = key > hi ? key : hi;
    });
    block_minmax(sm, lo, hi);
    block_select_bits<true>(sm, visit, r, lo, hi, 0, kth, kth_top, n_greater);
}

}  // namespace vts
