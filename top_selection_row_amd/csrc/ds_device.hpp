// ds_device.hpp -- gfx950 device building blocks of DeepSelect.
//
// * order-preserving keys of float32 / bfloat16 bit patterns
//   ("CUDA 算子笔记 4", milkfeng.top, section "改造 Radix Sort", float_to_key);
// * the random block order (SplitMix64 of Steele, Lea and Flood, OOPSLA 2014,
//   used as a counter-based hash; ids sorted by (hash, id));
// * RadixSelectTopK in LDS: MSD select over 8-bit digits with per-wave private
//   histograms ("改造 Radix Sort"; "并行算法（一）", elainafan.one, section
//   "Histogram" on privatisation), then an in-place stable partition keeping
//   the k largest (the predicate -> scan -> scatter "Compact" of
//   "并行算法（一）", done with 64-bit ballot masks and mbcnt ranks).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ds_plan.hpp"

namespace ds {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

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
// count <= 64*NW: rank counting -- wave w compares every id with the ids of its
// slice of the list and adds the partial ranks into LDS; then perm[rank] = id.
// Larger counts: a bitonic sort of (hash, id) pairs in LDS.
template <int NW>
__device__ void build_order(uint16_t* perm, uint64_t seed, int64_t row, int tag, int64_t id0, int count,
                            unsigned char* scratch) {
    constexpr int kLanes = NW * 64;
    const uint64_t ctr0 = ((uint64_t)(row * 2 + tag) << 32) + (uint64_t)id0;
    const int t = threadIdx.x, lane = lane_id(), wave = wave_id();
    uint64_t* hk = reinterpret_cast<uint64_t*>(scratch);
    if (count <= kLanes) {
        uint32_t* rank = reinterpret_cast<uint32_t*>(scratch + (size_t)count * 8);
        if (t < count) {
            hk[t] = splitmix_at(seed, ctr0 + (uint64_t)t);
            rank[t] = 0u;
        }
        __syncthreads();
        const int lo = wave * count / NW, hi = (wave + 1) * count / NW;
        for (int j = lane; j < count; j += 64) {
            const uint64_t h = hk[j];
            uint32_t r = 0;
            for (int i = lo; i < hi; ++i) {
                const uint64_t o = hk[i];
                r += (o < h) || (o == h && i < j);
            }
            if (r) atomicAdd(&rank[j], r);
        }
        __syncthreads();
        if (t < count) perm[rank[t]] = (uint16_t)t;
    } else {
        const int p2 = (int)next_pow2(count);
        uint32_t* hid = reinterpret_cast<uint32_t*>(scratch + (size_t)p2 * 8);
        for (int i = t; i < p2; i += kLanes) {
            hk[i] = i < count ? splitmix_at(seed, ctr0 + (uint64_t)i) : ~0ull;
            hid[i] = (uint32_t)i;
        }
        __syncthreads();
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
                __syncthreads();
            }
        }
        for (int i = t; i < count; i += kLanes) perm[i] = (uint16_t)hid[i];
    }
    __syncthreads();
}

// ----------------------------------------------------------------------------
// Workgroup-cooperative append (one tile spread over all waves): wave counts
// from the ballot masks, a prefix over the NW waves through LDS (one barrier),
// then each survivor's slot from mbcnt. `put(slot, pos)` stores slot's element
// at buffer position pos. Returns the number appended (uniform).
// ----------------------------------------------------------------------------
template <int NW, int NS, class Put>
__device__ __forceinline__ uint32_t append_masked(const uint64_t (&masks)[NS], const bool (&pred)[NS],
                                                  uint32_t len, uint32_t* cnt, uint32_t& par, Put&& put) {
    uint32_t c = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) c += (uint32_t)__popcll(masks[s]);
    const int wave = wave_id();
    if (lane_id() == 0) cnt[par * NW + wave] = c;
    __syncthreads();
    uint32_t base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t cw = cnt[par * NW + w];
        base += w < wave ? cw : 0u;
        total += cw;
    }
    par ^= 1u;
    total = uniform(total);
    if (c != 0) {
        uint32_t off = len + base;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if (pred[s]) put(s, off + lanes_below(masks[s]));
            off += (uint32_t)__popcll(masks[s]);
        }
    }
    return total;
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
// Histograms: one shared set of kHistCopies copies of the 256 bins, bin-major
// (word b*16 + c is copy c of bin b); lane l adds into copy l % 16. Lanes that
// share a bin therefore hit at most 4 words, and the 16 copies of a bin sit in
// 16 different LDS banks, so an atomic wave instruction costs at most a few
// conflict cycles even when every key falls into one bin (LDS atomics
// serialise per word). After the atomics the workgroup folds the copies into
// a compact 256-bin array, clearing them on the way.
// ----------------------------------------------------------------------------
constexpr int kHistCopies = 16;
constexpr int kHistWords = 256 * kHistCopies;  // plus 256 words of folded bins after them

struct SelectScratch {
    uint32_t* hist;  // kHistWords copies, then 256 folded bins
    uint32_t* pcnt;  // 2 x NW x 2
};

// Clear every histogram copy (each thread its share; caller adds the barrier).
template <int NW>
__device__ __forceinline__ void clear_hist(uint32_t* hist) {
    u32x4* h = reinterpret_cast<u32x4*>(hist);
    for (int i = threadIdx.x; i < kHistWords / 4; i += NW * 64) h[i] = u32x4{0u, 0u, 0u, 0u};
}

// Fold the copies into folded[256] and clear them (caller adds the barriers).
template <int NW>
__device__ __forceinline__ void fold_hist(uint32_t* hist) {
    constexpr int kPer = kHistWords / (NW * 64);  // words per thread (multiple of 4)
    static_assert(kHistWords % (NW * 64 * 4) == 0, "fold split");
    constexpr int kThreadsPerBin = kHistCopies / kPer;
    u32x4* h = reinterpret_cast<u32x4*>(hist) + threadIdx.x * (kPer / 4);
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < kPer / 4; ++j) {
        const u32x4 v = h[j];
        sum += v.x + v.y + v.z + v.w;
        h[j] = u32x4{0u, 0u, 0u, 0u};
    }
    if constexpr (kThreadsPerBin == 2) sum += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sum, 0x111, 0xF, 0xF, true);
    if constexpr (kThreadsPerBin == 4) {
        sum += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sum, 0x111, 0xF, 0xF, true);
        sum += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sum, 0x112, 0xF, 0xF, true);
    }
    if ((threadIdx.x % kThreadsPerBin) == kThreadsPerBin - 1) hist[kHistWords + threadIdx.x / kThreadsPerBin] = sum;
}

// Stable in-place partition of keys/idx[0, n): keep every key > kth and the
// first `need` keys == kth in buffer order, packed into [0, k). Rounds of
// 64*NW*R entries: each wave reads its 64*R entries into registers and
// publishes (greater, tied) counts; after one barrier every destination is
// known and lies at or before its source, so no round overwrites an entry
// that is still to be read.
template <class KeyT, int NW, int R = 8>
__device__ void partition_keep(KeyT* keys, uint32_t* idx, uint32_t n, uint32_t kth, uint32_t need,
                               uint32_t* pcnt) {
    const int lane = lane_id(), wave = wave_id();
    uint32_t sel_run = 0, tie_run = 0, par = 0;
    for (uint32_t base = 0; base < n; base += NW * 64 * R) {
        const uint32_t wbase = base + (uint32_t)wave * 64u * R;
        uint32_t kk[R], ii[R];
        uint64_t gm[R], tm[R];
        uint32_t g = 0, t = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t pos = wbase + (uint32_t)r * 64u + (uint32_t)lane;
            const bool v = pos < n;
            kk[r] = v ? (uint32_t)keys[pos] : 0u;
            ii[r] = v ? idx[pos] : 0u;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t pos = wbase + (uint32_t)r * 64u + (uint32_t)lane;
            const bool v = pos < n;
            gm[r] = __ballot(v & (kk[r] > kth));
            tm[r] = __ballot(v & (kk[r] == kth));
            g += (uint32_t)__popcll(gm[r]);
            t += (uint32_t)__popcll(tm[r]);
        }
        if (lane == 0) {
            pcnt[(par * NW + wave) * 2 + 0] = g;
            pcnt[(par * NW + wave) * 2 + 1] = t;
        }
        __syncthreads();
        uint32_t sel_before = sel_run, tie_before = tie_run, sel_round = 0, tie_round = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const uint32_t gw = uniform(pcnt[(par * NW + w) * 2 + 0]);
            const uint32_t tw = uniform(pcnt[(par * NW + w) * 2 + 1]);
            const uint32_t prior = tie_run + tie_round;
            const uint32_t room = need > prior ? need - prior : 0u;
            const uint32_t sw = gw + (tw < room ? tw : room);
            if (w < wave) {
                sel_before += sw;
                tie_before += tw;
            }
            sel_round += sw;
            tie_round += tw;
        }
        par ^= 1u;
        uint32_t sb = sel_before, tb = tie_before;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t pos = wbase + (uint32_t)r * 64u + (uint32_t)lane;
            const bool v = pos < n;
            const bool is_gt = v & (kk[r] > kth);
            const bool is_tie = v & (kk[r] == kth);
            const bool sel = is_gt | (is_tie & (tb + lanes_below(tm[r]) < need));
            const uint64_t sm = __ballot(sel);
            if (sel) {
                const uint32_t dst = sb + lanes_below(sm);
                keys[dst] = (KeyT)kk[r];
                idx[dst] = ii[r];
            }
            tb += (uint32_t)__popcll(tm[r]);
            sb += (uint32_t)__popcll(sm);
        }
        sel_run += sel_round;
        tie_run += tie_round;
    }
}

// Histogram of the digit (key >> shift) & 255 of every key of keys[0, n) that
// matches `prefix` under `pmask`. Keys are read 16 bytes at a time (4 or 8
// keys per lane) so the LDS reads pipeline; lane l adds into copy l % 16.
template <class KeyT, int NW>
__device__ __forceinline__ void histogram_pass(const KeyT* keys, uint32_t n, uint32_t prefix, uint32_t pmask,
                                               int shift, uint32_t* hist) {
    constexpr int kPer = 16 / sizeof(KeyT);
    uint32_t* hc = hist + (lane_id() & (kHistCopies - 1));
    const uint32_t nvec = n / kPer;
    const u32x4* kv = reinterpret_cast<const u32x4*>(keys);
    for (uint32_t i = threadIdx.x; i < nvec; i += NW * 64) {
        const u32x4 v = kv[i];
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            uint32_t key;
            if constexpr (sizeof(KeyT) == 4)
                key = v[q];
            else
                key = (v[q >> 1] >> ((q & 1) * 16)) & 0xFFFFu;
            if ((key & pmask) == prefix) atomicAdd(&hc[((key >> shift) & 0xFFu) * kHistCopies], 1u);
        }
    }
    for (uint32_t i = nvec * kPer + threadIdx.x; i < n; i += NW * 64) {
        const uint32_t key = keys[i];
        if ((key & pmask) == prefix) atomicAdd(&hc[((key >> shift) & 0xFFu) * kHistCopies], 1u);
    }
}

// Keep the k largest of keys/idx[0, n) (n > k) in [0, k); return the k-th key.
// MSD select over 8-bit digits: each pass histograms the digit of every key
// that matches the prefix fixed so far, folds the copies, and every wave walks
// the folded bins from the top to the one holding the rank-th largest (a
// 64-lane DPP prefix scan over the bins in descending order plus a 4-bin
// step). Passes start at the highest bit where the smallest and largest
// possible key (lo_key, *hi_ptr) differ: higher bits are shared by all keys.
// The histogram copies must be clear on entry; they are clear on return.
template <class D, int NW>
__device__ uint32_t radix_select(typename D::Key* keys, uint32_t* idx, uint32_t n, uint32_t k, SelectScratch& sc,
                                 uint32_t lo_key, const uint32_t* hi_ptr) {
    const int lane = lane_id();
    __syncthreads();  // every append / earlier partition is visible
    const uint32_t hi_key = uniform(*hi_ptr);
    const uint32_t diff = lo_key ^ (hi_key > lo_key ? hi_key : lo_key);
    const int top = diff ? 31 - __clz(diff) : 0;  // highest differing bit
    // first window [top-7, top] (clamped at 0); shared bits above it are fixed
    int shift = top >= 7 ? top - 7 : 0;
    uint32_t pmask = (shift + 8 >= 32) ? 0u : ~((1u << (shift + 8)) - 1u);
    uint32_t prefix = lo_key & pmask, rank = k;
    const uint32_t* folded = sc.hist + kHistWords;
    while (true) {
        histogram_pass<typename D::Key, NW>(keys, n, prefix, pmask, shift, sc.hist);
        __syncthreads();
        fold_hist<NW>(sc.hist);
        __syncthreads();
        // lane l holds bins 4*(63-l) .. 4*(63-l)+3, so a prefix sum over lanes
        // counts the keys in the bins from the top down to this lane's lowest
        const u32x4 c = reinterpret_cast<const u32x4*>(folded)[63 - lane];
        const uint32_t s = c.x + c.y + c.z + c.w;
        const uint32_t incl = wave_prefix_sum(s);
        const uint64_t ge = __ballot(incl >= rank);
        const int L = __builtin_ctzll(ge);  // first lane (from the top bins) reaching rank
        const int g = 63 - L;               // its bin group
        uint32_t above_cnt = uniform(__builtin_amdgcn_readlane(incl - s, L));
        const uint32_t c3 = uniform(__builtin_amdgcn_readlane(c.w, L));
        const uint32_t c2 = uniform(__builtin_amdgcn_readlane(c.z, L));
        const uint32_t c1 = uniform(__builtin_amdgcn_readlane(c.y, L));
        uint32_t d;
        if (above_cnt + c3 >= rank) {
            d = 4u * g + 3u;
        } else if (above_cnt + c3 + c2 >= rank) {
            above_cnt += c3;
            d = 4u * g + 2u;
        } else if (above_cnt + c3 + c2 + c1 >= rank) {
            above_cnt += c3 + c2;
            d = 4u * g + 1u;
        } else {
            above_cnt += c3 + c2 + c1;
            d = 4u * g;
        }
        rank -= above_cnt;
        prefix |= d << shift;
        pmask |= 0xFFu << shift;
        if (shift == 0) break;
        // next window; when it reaches below bit 8 it is [0, 7] and may overlap
        // bits already fixed -- every matching key agrees on those bits, so the
        // histogram and the prefix stay consistent
        shift = shift >= 8 ? shift - 8 : 0;
        __syncthreads();  // every wave has read the folded bins
    }
    partition_keep<typename D::Key, NW>(keys, idx, n, prefix, rank, sc.pcnt);
    return prefix;
}

}  // namespace ds
