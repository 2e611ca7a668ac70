// vts_device.hpp -- device building blocks for the top-k kernels (gfx950, wave64).
//
//  * order-preserving unsigned keys for fp32 / bf16 / fp16;
//  * wave64 ballot / mbcnt helpers and wave-aggregated LDS counters;
//  * a workgroup radix select (8-bit digits, LDS histogram, scan over the
//    256 bins) that finds the exact r-th largest key of any key set that the
//    workgroup can enumerate.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vts {

constexpr int NT = 256;               // threads per workgroup: 4 wave64
constexpr int WAVES = NT / 64;
constexpr int CAP = 4096;             // on-chip candidate slots per workgroup
constexpr int SAMPLE = 4096;          // sampled keys per row: 64 blocks of 64 columns
constexpr int SAMPLE_BLOCK = 64;
constexpr int SAMPLE_BLOCKS = SAMPLE / SAMPLE_BLOCK;
constexpr int SPT = SAMPLE / NT;      // sampled keys per thread (16)
constexpr int MAX_SPLIT = 32;         // workgroups per row, at most
constexpr int U = 4;                  // 16-byte vectors per thread per streaming step

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
__device__ __forceinline__ uint32_t gatomic_add(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add((VTS_GLOBAL uint32_t*)p, v, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
}

template <int DT> struct Traits;
template <> struct Traits<F32> {
    using raw_t = uint32_t;
    static constexpr int BITS = 32;
    static constexpr int VE = 4;  // elements per 16-byte vector
    static constexpr uint32_t PAD = 0xFF7FFFFFu;  // -FLT_MAX
};
template <> struct Traits<BF16> {
    using raw_t = uint16_t;
    static constexpr int BITS = 16;
    static constexpr int VE = 8;
    static constexpr uint32_t PAD = 0xFF7Fu;  // lowest finite bf16
};
template <> struct Traits<F16> {
    using raw_t = uint16_t;
    static constexpr int BITS = 16;
    static constexpr int VE = 8;
    static constexpr uint32_t PAD = 0xFBFFu;  // lowest finite fp16
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

// Shared state of one workgroup.
struct Smem {
    uint32_t key[CAP];
    uint32_t idx[CAP];
    uint32_t hist[256];
    uint32_t wsum[WAVES];
    uint32_t seg_cnt[MAX_SPLIT];
    uint32_t cand_n;
    uint32_t cnt_a, cnt_b;
    uint32_t sel_digit, sel_above;
    uint32_t flag;
    uint32_t total;
};

// Inclusive prefix sum over the workgroup (thread order).  Contains barriers:
// every thread must call it.
__device__ __forceinline__ uint32_t block_inclusive_scan(Smem& sm, uint32_t v) {
    const uint32_t lane = lane_id();
    const uint32_t w = threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t o = __shfl_up(v, d, 64);
        if (lane >= (uint32_t)d) v += o;
    }
    if (lane == 63) sm.wsum[w] = v;
    __syncthreads();
    uint32_t add = 0;
#pragma unroll
    for (int i = 0; i < WAVES; ++i)
        if ((uint32_t)i < w) add += sm.wsum[i];
    __syncthreads();
    return v + add;
}

// Workgroup sum of v.  Also returns, in cand_snapshot, the value of sm.cand_n
// read while no thread can change it (between the two barriers), so every
// thread takes the same decision on it.
__device__ __forceinline__ uint32_t block_sum(Smem& sm, uint32_t v, uint32_t& cand_snapshot) {
    uint32_t incl = block_inclusive_scan(sm, v);
    if (threadIdx.x == NT - 1) sm.total = incl;
    __syncthreads();
    const uint32_t t = sm.total;
    cand_snapshot = sm.cand_n;
    __syncthreads();
    return t;
}

// Exact r-th largest key (1-based rank r) of the key set that `visit`
// enumerates, by MSB-first 8-bit radix select.  visit(f) must call f(key) once
// for every key this thread owns (any order, any divergence).  The set must
// hold at least r keys.  Returns the key K and, in n_greater, how many keys of
// the set are strictly greater than K (so r - n_greater of the keys equal to K
// complete the top r).  Every thread must call it; contains barriers.
template <int BITS, class Visit>
__device__ __forceinline__ void block_select(Smem& sm, Visit visit, uint32_t r, uint32_t& kth,
                                             uint32_t& n_greater) {
    uint32_t prefix = 0, mask = 0, krem = r, gt = 0;
#pragma unroll
    for (int shift = BITS - 8; shift >= 0; shift -= 8) {
        sm.hist[threadIdx.x] = 0;
        __syncthreads();
        visit([&](uint32_t key) {
            if ((key & mask) == prefix) atomicAdd(&sm.hist[(key >> shift) & 0xFFu], 1u);
        });
        __syncthreads();
        // thread t holds bin 255 - t, so an inclusive scan counts keys in bins >= 255 - t
        const uint32_t b = 255u - threadIdx.x;
        const uint32_t v = sm.hist[b];
        const uint32_t incl = block_inclusive_scan(sm, v);
        const uint32_t excl = incl - v;
        if (excl < krem && incl >= krem) {
            sm.sel_digit = b;
            sm.sel_above = excl;
        }
        __syncthreads();
        const uint32_t d = sm.sel_digit, above = sm.sel_above;
        gt += above;
        krem -= above;
        prefix |= d << shift;
        mask |= 0xFFu << shift;
    }
    kth = prefix;
    n_greater = gt;
}

}  // namespace vts
