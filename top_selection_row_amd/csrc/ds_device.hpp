// ds_device.hpp -- gfx950 device building blocks of DeepSelect.
//
// * order-preserving keys of float32 / bfloat16 bit patterns
//   ("CUDA 算子笔记 4", milkfeng.top, section "改造 Radix Sort", float_to_key);
// * the random block order (SplitMix64 of Steele, Lea and Flood, OOPSLA 2014,
//   used as a counter-based hash; ids sorted by (hash, id));
// * RadixSelectTopK in LDS: MSD select over 8-bit digits with privatised
//   histograms ("改造 Radix Sort"; "并行算法（一）", elainafan.one, section
//   "Histogram" on privatisation), then an in-place stable partition keeping
//   the k largest (the predicate -> scan -> scatter "Compact" of
//   "并行算法（一）", with DPP prefix sums inside a wave).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ds_plan.hpp"

namespace ds {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Workgroup barrier for LDS traffic: waits for this wave's LDS operations
// only. __syncthreads() also waits for every outstanding vector-memory
// operation, which would stall each step on the ring's prefetches into LDS;
// no kernel here exchanges global memory between its waves, and each wave
// waits (vmcnt) for its own ring blocks before it reads them.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Number of set bits of m in the lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// ----------------------------------------------------------------------------
// Keys. A pattern with its sign bit set has every bit flipped, otherwise only
// its sign bit: unsigned key order is float order, -0 < +0, NaNs outermost.
// ----------------------------------------------------------------------------
__device__ __forceinline__ uint32_t key_f32(uint32_t u) {
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ uint32_t raw_f32(uint32_t key) {
    return key ^ ((uint32_t)((int32_t)~key >> 31) | 0x80000000u);
}
__device__ __forceinline__ uint32_t key_bf16(uint32_t u16) {
    return (u16 ^ ((uint32_t)((int32_t)(u16 << 16) >> 31) | 0x8000u)) & 0xFFFFu;
}
__device__ __forceinline__ uint32_t raw_bf16(uint32_t key16) {
    return (key16 ^ ((uint32_t)((int32_t)(~key16 << 16) >> 31) | 0x8000u)) & 0xFFFFu;
}

struct F32T {
    using Key = uint32_t;
    static constexpr int kBits = 32;
    static constexpr int kBytes = 4;
    static constexpr int kPerLoad = 4;  // elements in one 16-byte load
    __device__ static uint32_t key(uint32_t raw) { return key_f32(raw); }
    __device__ static uint32_t raw(uint32_t key) { return raw_f32(key); }
};
struct BF16T {
    using Key = uint16_t;
    static constexpr int kBits = 16;
    static constexpr int kBytes = 2;
    static constexpr int kPerLoad = 8;
    __device__ static uint32_t key(uint32_t raw) { return key_bf16(raw); }
    __device__ static uint32_t raw(uint32_t key) { return raw_bf16(key); }
};

// bfloat16 candidates packed with their part-local column into one 32-bit
// entry, key << 16 | column (parts of at most 65536 elements): one LDS store
// per candidate instead of two. The select reads the key from the top half
// and moves whole entries.
struct BF16P {
    using Key = uint32_t;
    static constexpr int kBits = 16;
    static constexpr int kBytes = 2;
    static constexpr int kPerLoad = 8;
    __device__ static uint32_t key(uint32_t raw) { return key_bf16(raw); }
    __device__ static uint32_t raw(uint32_t key) { return raw_bf16(key); }
};
template <class D>
struct is_packed {
    static constexpr bool value = false;
};
template <>
struct is_packed<BF16P> {
    static constexpr bool value = true;
};

// Threshold test on raw bits, exact under the key order:
//   T >= +0 : key(x) > key(T)  <=>  (int)x > (int)t
//   T <  0  : key(x) > key(T)  <=>  (unsigned)x < (unsigned)t
// For bfloat16 the 16-bit pattern sits in the top half of a 32-bit word w and
// thr = t<<16 (T < 0) or t<<16 | 0xFFFF (T >= +0), so one 32-bit compare
// decides it whatever the low half holds.
struct Thresh {
    bool neg;
    uint32_t thr;
};
template <class D>
__device__ __forceinline__ Thresh make_thresh(uint32_t tkey) {
    Thresh t;
    if constexpr (D::kBytes == 4) {
        t.neg = tkey < 0x80000000u;
        t.thr = D::raw(tkey);
    } else {
        t.neg = tkey < 0x8000u;
        const uint32_t r = D::raw(tkey) << 16;
        t.thr = t.neg ? r : (r | 0xFFFFu);
    }
    return t;
}
__device__ __forceinline__ bool above(uint32_t w, const Thresh& t) {
    return t.neg ? (w < t.thr) : ((int32_t)w > (int32_t)t.thr);
}
// The same test with the sign of T fixed at compile time (one compare).
template <bool kNeg>
__device__ __forceinline__ bool above_k(uint32_t w, uint32_t thr) {
    if constexpr (kNeg)
        return w < thr;
    else
        return (int32_t)w > (int32_t)thr;
}

// ----------------------------------------------------------------------------
// Block order: counter c -> SplitMix64 output number c for `seed` (state
// seed + (c+1)*gamma, then the variant-13 mix). Ids sorted by (hash, id).
// ----------------------------------------------------------------------------
__device__ __forceinline__ uint64_t splitmix_at(uint64_t seed, uint64_t ctr) {
    uint64_t z = seed + (ctr + 1ull) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// perm[i] = the i-th of `count` ids (0-based, relative to id0) in random order.
// Every thread of the workgroup must call it; it ends with a barrier.
// count <= 64*NW: rank counting -- thread t counts the hashes below id t's
// and writes perm[rank] = t. Larger counts: a bitonic sort of (hash, id)
// pairs in LDS.
template <int NW>
__device__ void build_order(uint16_t* perm, uint64_t seed, int64_t row, int tag, int64_t id0, int count,
                            unsigned char* scratch) {
    constexpr int kLanes = NW * 64;
    const uint64_t ctr0 = ((uint64_t)(row * 2 + tag) << 32) + (uint64_t)id0;
    const int t = threadIdx.x, lane = lane_id(), wave = wave_id();
    uint64_t* hk = reinterpret_cast<uint64_t*>(scratch);
    if (count <= kLanes) {
        // Hashes of distinct ids differ (SplitMix64's state steps by an odd
        // constant and each step of its mix is a bijection of 64-bit words),
        // so an id's place is the number of smaller hashes: thread t counts
        // them for id t over the whole list, read 8 hashes at a time (16-byte
        // broadcast reads; the list is padded to a multiple of 8 with the
        // largest word, which is smaller than no hash).
        const int padded = (count + 7) & ~7;
        const uint64_t h = t < count ? splitmix_at(seed, ctr0 + (uint64_t)t) : 0ull;
        if (t < padded) hk[t] = t < count ? h : ~0ull;
        lds_barrier();
        if (t < count) {
            const u32x4* hv = reinterpret_cast<const u32x4*>(hk);
            uint32_t r = 0;
            for (int i0 = 0; i0 < padded; i0 += 8) {
                u32x4 v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = hv[i0 / 2 + q];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint64_t a = ((uint64_t)v[q].y << 32) | v[q].x;
                    const uint64_t b = ((uint64_t)v[q].w << 32) | v[q].z;
                    r += (a < h ? 1u : 0u) + (b < h ? 1u : 0u);
                }
            }
            perm[r] = (uint16_t)t;
        }
    } else {
        const int p2 = (int)next_pow2(count);
        uint32_t* hid = reinterpret_cast<uint32_t*>(scratch + (size_t)p2 * 8);
        for (int i = t; i < p2; i += kLanes) {
            hk[i] = i < count ? splitmix_at(seed, ctr0 + (uint64_t)i) : ~0ull;
            hid[i] = (uint32_t)i;
        }
        lds_barrier();
        for (int size = 2; size <= p2; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int i = t; i < p2; i += kLanes) {
                    const int j = i ^ stride;
                    if (j > i) {
                        const uint64_t a = hk[i], b = hk[j];
                        const uint32_t ia = hid[i], ib = hid[j];
                        const bool a_gt = a > b || (a == b && ia > ib);
                        if (a_gt == ((i & size) == 0)) {
                            hk[i] = b;
                            hk[j] = a;
                            hid[i] = ib;
                            hid[j] = ia;
                        }
                    }
                }
                lds_barrier();
            }
        }
        for (int i = t; i < count; i += kLanes) perm[i] = (uint16_t)hid[i];
    }
    lds_barrier();
}

// Largest value over the wave, returned uniform (a DPP max scan whose last
// lane holds the maximum; lanes outside a move contribute 0).
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
    uint32_t o;
    o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);
    v = o > v ? o : v;
    o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);
    v = o > v ? o : v;
    o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);
    v = o > v ? o : v;
    o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);
    v = o > v ? o : v;
    o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);
    v = o > v ? o : v;
    o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);
    v = o > v ? o : v;
    return uniform(__builtin_amdgcn_readlane(v, 63));
}

// Smallest value over the wave, returned uniform (the largest complement).
__device__ __forceinline__ uint32_t wave_min(uint32_t v) { return ~wave_max(~v); }

// Inclusive prefix sum over the 64 lanes (lane l gets the sum over lanes <= l)
// with DPP moves only: shifts by 1, 2, 4 and 8 inside each row of 16 lanes,
// then the last lane of row 0 (2) is added to row 1 (3) and the last lane of
// row 1 to rows 2 and 3. No LDS round trip.
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false); // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false); // row_bcast:31
    return v;
}

// ----------------------------------------------------------------------------
// RadixSelectTopK in LDS.
//
// The candidates are read in chunks of 8 consecutive entries: chunk c covers
// entries [8c, 8c+8) and round r of a workgroup of NT threads gives chunk
// r*NT + t to thread t. Keys are read 16 bytes at a time.
//
// Digits are relative to the range the keys are known to lie in: a pass over
// keys in [base, base+span] uses digit (key - base) >> s, s the smallest shift
// that leaves at most 256 digits, so a pass resolves 8 bits of the span rather
// than 8 fixed bits of the key (once T is set the span is the distance from T
// to the largest key appended, often under 256).
//
// Histograms: 16 copies of 256 16-bit counters, two bins per word; lane l adds
// into copy l % 16, word (d / 2) * 16 + l % 16. The 16 copies of a word sit in
// 16 different banks, so lanes that share a digit hit at most 4 words of it.
// A fold sums the copies into 256 bins and clears them.
// ----------------------------------------------------------------------------
constexpr uint32_t kHistCopies = 16;
constexpr uint32_t kHistWords = 128 * kHistCopies;  // 8 KiB

template <class D>
struct KeyChunk {
    u32x4 v[sizeof(typename D::Key) == 4 ? 2 : 1];
};

template <class D>
__device__ __forceinline__ void read_chunk(KeyChunk<D>& kc, const typename D::Key* keys, uint32_t c) {
    constexpr uint32_t W = sizeof(typename D::Key) == 4 ? 2u : 1u;
    const u32x4* kv = reinterpret_cast<const u32x4*>(keys) + c * W;
    kc.v[0] = kv[0];
    if constexpr (W == 2) kc.v[1] = kv[1];
}

// Key of entry i of a chunk, and the entry as stored (the same but for
// packed entries, whose key is the top half).
template <class D>
__device__ __forceinline__ uint32_t chunk_key(const KeyChunk<D>& kc, int i) {
    if constexpr (is_packed<D>::value)
        return kc.v[i >> 2][i & 3] >> 16;
    else if constexpr (D::kBytes == 4)
        return kc.v[i >> 2][i & 3];
    else
        return (kc.v[0][i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
}
template <class D>
__device__ __forceinline__ uint32_t chunk_entry(const KeyChunk<D>& kc, int i) {
    if constexpr (sizeof(typename D::Key) == 4)
        return kc.v[i >> 2][i & 3];
    else
        return (kc.v[0][i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
}

// Clear `words` words of LDS (each thread its share; caller adds the barrier).
template <int NW>
__device__ __forceinline__ void clear_words(uint32_t* p, uint32_t words) {
    u32x4* h = reinterpret_cast<u32x4*>(p);
    for (uint32_t i = threadIdx.x; i < words / 4; i += NW * 64) h[i] = u32x4{0u, 0u, 0u, 0u};
}

// Add every key of keys[0, n) with key - base <= span into the digit
// (key - base) >> s of this lane's histogram copy (16-bit counts, two bins a
// word). Lanes whose key is outside the window do not add; a chunk's keys are
// checked against the end of the buffer only in the round that holds it, and
// the next round's chunk is read before this one is counted.
template <class D, int NW, bool kFull, bool kAll>
__device__ __forceinline__ void hist_chunk(const KeyChunk<D>& kc, uint32_t lim, uint32_t base, uint32_t span, int s,
                                           uint32_t* hl) {
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        const uint32_t u = chunk_key<D>(kc, i) - base;
        // bin pair (digit >> 1) and half (digit & 1) by bit-field extracts
        uint32_t* at = &hl[__builtin_amdgcn_ubfe(u, (uint32_t)(s + 1), 7u) * kHistCopies];
        const uint32_t inc = 1u + __builtin_amdgcn_ubfe(u, (uint32_t)s, 1u) * 0xFFFFu;
        if constexpr (kAll)
            atomicAdd(at, (kFull || (uint32_t)i < lim) ? inc : 0u);
        else if ((kFull || (uint32_t)i < lim) && u <= span)
            atomicAdd(at, inc);
    }
}

// kAll: every key of the buffer lies in the window (the first pass of a
// select), so no lane skips its add.
template <class D, int NW, bool kAll>
__device__ __forceinline__ void hist_pass(const typename D::Key* keys, uint32_t n, uint32_t base, uint32_t span,
                                          int s, uint32_t* hist) {
    constexpr uint32_t NT = NW * 64;
    const uint32_t nch = (n + kChunk - 1) / kChunk;
    uint32_t* hl = hist + (lane_id() & (kHistCopies - 1));
    uint32_t c = threadIdx.x;
    KeyChunk<D> kc;
    read_chunk<D>(kc, keys, c < nch ? c : 0u);
    for (uint32_t c0 = 0; c0 < nch; c0 += NT, c += NT) {
        KeyChunk<D> nx = kc;
        if (c0 + NT < nch) read_chunk<D>(nx, keys, c + NT < nch ? c + NT : 0u);  // the next round's chunk
        const uint32_t lim = c < nch ? n - c * kChunk : 0u;
        if (__ballot(lim < (uint32_t)kChunk) == 0ull)
            hist_chunk<D, NW, true, kAll>(kc, lim, base, span, s, hl);
        else
            hist_chunk<D, NW, false, kAll>(kc, lim, base, span, s, hl);
        kc = nx;
    }
}

// Fold the copies into folded[256] and clear them (caller adds barriers).
// Thread t sums the words [4t, 4t+4) (or [8t, 8t+8) with 4 waves): copies of
// bins 2g and 2g+1, g = word / 16; the threads of a group combine with DPP
// shifts and the last of them writes the two bins.
template <int NW>
__device__ __forceinline__ void fold_pass(uint32_t* hist, uint32_t* folded) {
    constexpr int NT = NW * 64;
    constexpr int WPT = kHistWords / NT;      // words per thread (2, 4 or 8)
    constexpr int TPG = kHistCopies / WPT;    // threads per group (8, 4 or 2)
    static_assert((WPT == 2 || WPT % 4 == 0) && TPG >= 1 && TPG <= 8, "fold split");
    const int t = threadIdx.x, g = t / TPG;
    uint32_t a = 0, b = 0;
    if constexpr (WPT == 2) {
        uint2* h = reinterpret_cast<uint2*>(hist) + t;
        const uint2 v = *h;
        a = (v.x & 0xFFFFu) + (v.y & 0xFFFFu);
        b = (v.x >> 16) + (v.y >> 16);
        *h = uint2{0u, 0u};
    } else {
        u32x4* h = reinterpret_cast<u32x4*>(hist) + t * (WPT / 4);
#pragma unroll
        for (int j = 0; j < WPT / 4; ++j) {
            const u32x4 v = h[j];
            a += (v.x & 0xFFFFu) + (v.y & 0xFFFFu) + (v.z & 0xFFFFu) + (v.w & 0xFFFFu);
            b += (v.x >> 16) + (v.y >> 16) + (v.z >> 16) + (v.w >> 16);
            h[j] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    if constexpr (TPG >= 2) {
        a += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x111, 0xF, 0xF, true);
        b += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)b, 0x111, 0xF, 0xF, true);
    }
    if constexpr (TPG >= 4) {
        a += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x112, 0xF, 0xF, true);
        b += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)b, 0x112, 0xF, 0xF, true);
    }
    if constexpr (TPG >= 8) {
        a += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x114, 0xF, 0xF, true);
        b += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)b, 0x114, 0xF, 0xF, true);
    }
    if (t % TPG == TPG - 1) reinterpret_cast<uint2*>(folded)[g] = uint2{a, b};
}

// The bin of folded[256] that holds the rank-th largest key (every wave, same
// answer): lane l takes bins 4*(63-l) .. 4*(63-l)+3, a prefix sum over lanes
// counts the keys from the top bin down, the first lane reaching rank names
// the group and a 4-bin step the bin. rank becomes the rank inside that bin,
// count the number of keys in it.
__device__ __forceinline__ uint32_t pick_bin(const uint32_t* folded, uint32_t& rank, uint32_t& count) {
    const int lane = lane_id();
    const u32x4 c = reinterpret_cast<const u32x4*>(folded)[63 - lane];
    const uint32_t s = c.x + c.y + c.z + c.w;
    const uint32_t incl = wave_prefix_sum(s);
    // every lane resolves its own 4 bins as if it held the rank-th key (vector
    // selects, no branches); the lane that does is read back once
    const uint32_t ex = incl - s;  // keys in the bins above this lane's
    const uint32_t a3 = ex + c.w, a2 = a3 + c.z, a1 = a2 + c.y;
    const bool h3 = a3 >= rank, h2 = a2 >= rank, h1 = a1 >= rank;
    const uint32_t j = h3 ? 3u : h2 ? 2u : h1 ? 1u : 0u;
    const uint32_t cnt = h3 ? c.w : h2 ? c.z : h1 ? c.y : c.x;
    const uint32_t abv = h3 ? ex : h2 ? a3 : h1 ? a2 : a1;
    const uint64_t ge = __ballot(incl >= rank);
    const int L = __builtin_ctzll(ge);
    count = uniform(__builtin_amdgcn_readlane(cnt, L));
    rank -= uniform(__builtin_amdgcn_readlane(abv, L));
    return 4u * (uint32_t)(63 - L) + uniform(__builtin_amdgcn_readlane(j, L));
}

// Stable in-place partition of keys/idx[0, n): keep every key > kth and the
// first `need` keys == kth, in buffer order, packed into [0, k). Groups of up
// to kRoundsPerGroup rounds: every thread marks the greater and the tied
// entries of its chunks in two 8-bit masks, a DPP prefix sum of their counts
// inside the wave and one LDS exchange of the wave totals (one barrier per
// group) give each chunk the number of kept entries before it, and each kept
// entry goes to that number plus the kept entries before it in the chunk (a
// bit count of the mask). A destination never passes the entry's own
// position, so no group overwrites an entry a later group still reads.
// Dropped entries are stored to a per-lane junk slot past the buffer, so the
// stores need no branch.
// Returns the number of entries kept (the same in every thread).
template <class D, int NW>
__device__ __forceinline__ uint32_t partition_keep(typename D::Key* keys, uint32_t* idx, uint32_t* tot, uint32_t n,
                                                   uint32_t kth, uint32_t need, uint32_t junk) {
    constexpr int NT = NW * 64, R = kRoundsPerGroup;
    const int t = threadIdx.x, lane = lane_id(), wave = wave_id();
    const uint32_t nch = (n + kChunk - 1) / kChunk;
    const uint32_t my_junk = junk + (uint32_t)lane;
    uint32_t run = 0, par = 0;  // greater | tied << 16 before this group
    for (uint32_t c0 = 0; c0 < nch; c0 += NT * R) {
        const int nr = nch - c0 > (uint32_t)NT ? R : 1;
        KeyChunk<D> kc[R];
        u32x4 ix[R][2];
        uint32_t gm[R], em[R], mine[R], incl[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r < nr) {
                const uint32_t c = c0 + r * NT + t;
                const bool has = c < nch;
                const uint32_t cr = has ? c : 0u;
                read_chunk<D>(kc[r], keys, cr);
                if constexpr (!is_packed<D>::value) {
                    const u32x4* iv = reinterpret_cast<const u32x4*>(idx) + cr * 2u;
                    ix[r][0] = iv[0];
                    ix[r][1] = iv[1];
                }
                const uint32_t lim = has ? n - c * kChunk : 0u;
                const uint32_t valid = lim >= (uint32_t)kChunk ? 0xFFu : ((1u << lim) - 1u);
                uint32_t g = 0, e = 0;
#pragma unroll
                for (int i = 0; i < kChunk; ++i) {
                    const uint32_t key = chunk_key<D>(kc[r], i);
                    g |= key > kth ? 1u << i : 0u;
                    e |= key == kth ? 1u << i : 0u;
                }
                gm[r] = g & valid;
                em[r] = e & valid;
                mine[r] = (uint32_t)__builtin_popcount(gm[r]) | ((uint32_t)__builtin_popcount(em[r]) << 16);
                incl[r] = wave_prefix_sum(mine[r]);
                if (lane == 63) tot[(par * R + r) * NW + wave] = incl[r];
            }
        }
        lds_barrier();
        const u32x4* tv = reinterpret_cast<const u32x4*>(tot + par * R * NW);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r < nr) {
                uint32_t before = run, all = 0;
#pragma unroll
                for (int w4 = 0; w4 < NW / 4; ++w4) {
                    const u32x4 x = tv[(r * NW) / 4 + w4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        before += (w4 * 4 + q < wave) ? x[q] : 0u;
                        all += x[q];
                    }
                }
                const uint32_t excl = before + incl[r] - mine[r];
                const uint32_t tie = excl >> 16;
                const uint32_t ne = mine[r] >> 16;
                // the tied entries of this chunk that are kept: the first
                // need - tie of them (all when they fit, none when need is reached)
                uint32_t ke = tie + ne <= need ? em[r] : 0u;
                if (__ballot(tie < need && tie + ne > need) != 0ull) {
                    if (tie < need && tie + ne > need) {
                        uint32_t left = need - tie, m = em[r];
                        for (int i = 0; i < kChunk; ++i) {
                            if (left != 0u && ((m >> i) & 1u)) {
                                ke |= 1u << i;
                                --left;
                            }
                        }
                    }
                }
                const uint32_t km = gm[r] | ke;
                const uint32_t dst0 = (excl & 0xFFFFu) + (tie < need ? tie : need);
#pragma unroll
                for (int i = 0; i < kChunk; ++i) {
                    const bool kp = (km >> i) & 1u;
                    const uint32_t at = kp ? (uint32_t)__builtin_popcount(km & ((1u << i) - 1u)) + dst0 : my_junk;
                    keys[at] = (typename D::Key)chunk_entry<D>(kc[r], i);
                    if constexpr (!is_packed<D>::value) idx[at] = ix[r][i >> 2][i & 3];
                }
                run += all;
            }
        }
        par ^= 1u;
    }
    const uint32_t tied = run >> 16;
    return (run & 0xFFFFu) + (tied < need ? tied : need);
}

// The rest of a select once the bin of the k-th key holds few keys: every
// key of keys[0, n) with key - base <= span is appended to gathered[] (a
// counter in *gcount, zero on entry), then after one barrier every wave
// resolves the remaining digits of the gathered keys alone, on its own
// 256-bin histogram (a quarter of the histogram copies, clear on entry and
// on return): no further barrier and no fold. Once the window holds a single
// key, or a pass keeps every gathered key and they are all equal, that key
// is the answer and no further pass runs.
template <class D, int NW>
__device__ __forceinline__ uint32_t finish_gathered(const typename D::Key* keys, uint32_t n, uint32_t base,
                                                    uint32_t span, int s, uint32_t& rank, uint32_t* hist,
                                                    uint32_t* gathered, uint32_t* gcount) {
    constexpr uint32_t NT = NW * 64;
    const uint32_t nch = (n + kChunk - 1) / kChunk;
    const int lane0 = lane_id();
    for (uint32_t c0 = 0; c0 < nch; c0 += NT) {
        const uint32_t c = c0 + threadIdx.x;
        KeyChunk<D> kc;
        read_chunk<D>(kc, keys, c < nch ? c : 0u);
        const uint32_t lim = c < nch ? n - c * kChunk : 0u;
        uint32_t m = 0;  // entries of this chunk in the window
#pragma unroll
        for (int i = 0; i < kChunk; ++i)
            m |= ((uint32_t)i < lim && chunk_key<D>(kc, i) - base <= span) ? 1u << i : 0u;
        // one counter update per wave: a lane prefix sum of the matches, the
        // last lane reserves the wave's slots
        const uint32_t cnt = (uint32_t)__builtin_popcount(m);
        const uint32_t incl = wave_prefix_sum(cnt);
        const uint32_t total = uniform(__builtin_amdgcn_readlane(incl, 63));
        if (total != 0u) {
            uint32_t at = 0;
            if (lane0 == 63) at = atomicAdd(gcount, total);
            at = uniform(__builtin_amdgcn_readlane(at, 63)) + incl - cnt;
#pragma unroll
            for (int i = 0; i < kChunk; ++i) {
                if ((m >> i) & 1u) {
                    if (at < (uint32_t)kGather) gathered[at] = chunk_key<D>(kc, i);
                    ++at;
                }
            }
        }
    }
    lds_barrier();
    const uint32_t ng = min(uniform(*gcount), (uint32_t)kGather);
    const int lane = lane_id();
    uint32_t g[kGather / 64];
#pragma unroll
    for (int j = 0; j < kGather / 64; ++j) g[j] = (uint32_t)(lane + 64 * j) < ng ? gathered[lane + 64 * j] : 0u;
    static_assert(NW * 256 <= (int)kHistWords, "a 256-bin histogram per wave must fit the histogram copies");
    uint32_t* wh = hist + wave_id() * 256;  // this wave's 256 bins
    uint32_t cnt = ng;     // keys in the window
    bool passed = false;   // a pass has narrowed the window
    while (s > 0) {
        if (passed && cnt == ng) {
            // the pass kept every gathered key (ties, mostly): when all of
            // them equal the first, that key is the k-th, and rank counts
            // the equal keys kept
            const uint32_t g0 = uniform(__builtin_amdgcn_readfirstlane(g[0]));
            bool other = false;
#pragma unroll
            for (int j = 0; j < kGather / 64; ++j) other |= (uint32_t)(lane + 64 * j) < ng && g[j] != g0;
            if (__ballot(other) == 0ull) return g0;
        }
        passed = true;
        if (cnt == 1u) {
            // one key left in the window: it is the k-th (rank is 1), and
            // the remaining digits are its own
            uint32_t mine = 0;
#pragma unroll
            for (int j = 0; j < kGather / 64; ++j)
                mine = (uint32_t)(lane + 64 * j) < ng && g[j] - base <= span ? g[j] : mine;
            return uniform(wave_max(mine));
        }
        s = s > 8 ? s - 8 : 0;
#pragma unroll
        for (int j = 0; j < kGather / 64; ++j) {
            const uint32_t u = g[j] - base;
            if ((uint32_t)(lane + 64 * j) < ng && u <= span) atomicAdd(&wh[(u >> s) & 255u], 1u);
        }
        const uint32_t d = pick_bin(wh, rank, cnt);
        reinterpret_cast<u32x4*>(wh)[lane] = u32x4{0u, 0u, 0u, 0u};
        base += d << s;
        span = (1u << s) - 1u;
    }
    return base;
}

// 16-bit keys spanning 256 to 4095 keys: one pass over a single histogram of
// kWideBins 16-bit counters (the copies' 8 KiB, two bins a word, bin
// key - base) finds the rank-th largest key, where digits of 256 bins take
// two passes. Thread t owns the words [WPT (NT - 1 - t), + WPT), so thread 0
// holds the top bins and an inclusive prefix of the threads' counts, taken
// in thread order, counts the keys from the top bin down; the thread whose
// bins hold the rank-th key names it, and the rank among the keys equal to
// it, in folded[0, 2). Every key of keys[0, n) must lie in the window and n
// must be under 2^16 (a counter holds a whole bin). The histogram is clear
// on entry and cleared as it is read; tot[0, NW) carries the waves' totals.
constexpr uint32_t kWideBins = 2 * kHistWords;

template <class D, int NW>
__device__ __forceinline__ uint32_t wide_pick(const typename D::Key* keys, uint32_t n, uint32_t base,
                                              uint32_t* hist, uint32_t* tot, uint32_t* folded, uint32_t& rank) {
    constexpr uint32_t NT = NW * 64, WPT = kHistWords / NT;
    static_assert(WPT % 4 == 0 && WPT * NT == kHistWords && kHistWords == 2048, "whole 16-byte reads of the histogram");
    const uint32_t nch = (n + kChunk - 1) / kChunk;
    for (uint32_t c = threadIdx.x; c < nch; c += NT) {
        KeyChunk<D> kc;
        read_chunk<D>(kc, keys, c);
        const uint32_t lim = n - c * kChunk;
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            const uint32_t u = chunk_key<D>(kc, i) - base;
            // word (u >> 1) masked to the histogram (u < kWideBins already)
            if ((uint32_t)i < lim) atomicAdd(&hist[__builtin_amdgcn_ubfe(u, 1u, 11u)], 1u << ((u & 1u) << 4));
        }
    }
    lds_barrier();
    const uint32_t w0 = WPT * (NT - 1u - threadIdx.x);
    uint32_t cw[WPT];
    uint32_t sum = 0;
    u32x4* h = reinterpret_cast<u32x4*>(hist + w0);
#pragma unroll
    for (uint32_t j = 0; j < WPT / 4; ++j) {
        const u32x4 v = h[j];
        h[j] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            cw[4 * j + q] = v[q];
            sum += (v[q] & 0xFFFFu) + (v[q] >> 16);
        }
    }
    const uint32_t incl = wave_prefix_sum(sum);
    if (lane_id() == 63) tot[wave_id()] = incl;
    lds_barrier();
    uint32_t above = incl - sum;  // keys in the bins above this thread's
#pragma unroll
    for (int v = 0; v < NW; ++v) above += v < wave_id() ? tot[v] : 0u;
    if (above < rank && above + sum >= rank) {
        uint32_t bin = 0, r = 0;
        bool found = false;
#pragma unroll
        for (int j = (int)WPT - 1; j >= 0; --j) {
#pragma unroll
            for (int half = 1; half >= 0; --half) {
                const uint32_t c = half ? cw[j] >> 16 : cw[j] & 0xFFFFu;
                if (!found && above + c >= rank) {
                    bin = 2u * (w0 + (uint32_t)j) + (uint32_t)half;
                    r = rank - above;
                    found = true;
                }
                above += c;
            }
        }
        folded[0] = bin;
        folded[1] = r;
    }
    lds_barrier();
    rank = uniform(folded[1]);
    return base + uniform(folded[0]);
}

// RadixSelectTopK: keep the k largest of keys/idx[0, n) (k <= n) in [0, k)
// and return the k-th largest key. Every key lies in [lo, hi]. Entries
// [junk, junk+64) of both arrays are scratch for dropped entries. Starts with a
// barrier (the caller's appends become visible) unless the caller has just
// passed one (synced); the histogram copies must be clear on entry and are
// clear on return.
// `mark(c)` is called after each phase (c: 5 entry, 6 histogram, 7 fold,
// 8 pick, 9 partition, 10 gathered finish): a cycle-accounting hook of the
// profiling build, nothing otherwise.
struct NoMark {
    __device__ void operator()(int) const {}
};
template <class D, int NW, class Mark = NoMark>
__device__ uint32_t select_topk(typename D::Key* keys, uint32_t* idx, uint32_t* hist, uint32_t* folded,
                                uint32_t* tot, uint32_t* gathered, uint32_t* gcount, uint32_t junk, uint32_t n,
                                uint32_t k, uint32_t lo, uint32_t hi, bool all_in = true, bool synced = false,
                                Mark mark = {}) {
    if (!synced) lds_barrier();  // synced: the caller's own barrier made the buffer visible
    mark(5);
    uint32_t base = lo, span = hi - lo, rank = k;
    if constexpr (D::kBits == 16) {
        if (all_in && span >= 256u && span < kWideBins && n < 65536u) {
            base = wide_pick<D, NW>(keys, n, lo, hist, tot, folded, rank);
            mark(6);
            partition_keep<D, NW>(keys, idx, tot, n, base, rank, junk);
            mark(9);
            return base;
        }
    }
    int s = span ? 32 - __clz(span) : 0;  // bit length of the span
    s = s > 8 ? s - 8 : 0;
    bool first = all_in;  // the first pass's window holds every key
    while (true) {
        if (first)
            hist_pass<D, NW, true>(keys, n, base, span, s, hist);
        else
            hist_pass<D, NW, false>(keys, n, base, span, s, hist);
        first = false;
        if (threadIdx.x == 0) *gcount = 0u;
        lds_barrier();
        mark(6);
        fold_pass<NW>(hist, folded);
        lds_barrier();
        mark(7);
        uint32_t cnt;
        base += pick_bin(folded, rank, cnt) << s;
        mark(8);
        if (s == 0) break;
        span = (1u << s) - 1u;
        // gathering pays off when two or more digits remain (32-bit keys);
        // for one more digit a plain pass is cheaper
        if constexpr (D::kBits > 16) {
            if (cnt <= (uint32_t)kGather && s > 8) {
                base = finish_gathered<D, NW>(keys, n, base, span, s, rank, hist, gathered, gcount);
                mark(10);
                break;
            }
        }
        s = s > 8 ? s - 8 : 0;
    }
    partition_keep<D, NW>(keys, idx, tot, n, base, rank, junk);
    mark(9);
    return base;
}

}  // namespace ds
