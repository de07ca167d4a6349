// ds_device.hpp -- gfx950 device building blocks of DeepSelect.
//
// * order-preserving keys of float32 / bfloat16 bit patterns
//   ("CUDA 算子笔记 4", milkfeng.top, section "改造 Radix Sort", float_to_key);
// * the random block order (SplitMix64 of Steele, Lea and Flood, OOPSLA 2014,
//   used as a counter-based hash, ids sorted by (hash, id));
// * wave64 ballot / mbcnt compaction and a workgroup prefix over 4 waves
//   (the predicate -> scan -> scatter "Compact" of "并行算法（一）",
//   elainafan.one, done with lane masks instead of a tree scan);
// * RadixSelectTopK in LDS: MSD select over 8-bit digits with per-wave private
//   histograms ("改造 Radix Sort"; "并行算法（一）" section "Histogram" on
//   privatisation), then an in-place stable partition keeping the k largest.
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

// ----------------------------------------------------------------------------
// Block order: counter c -> SplitMix64 output number c for `seed` (state seed +
// (c+1)*gamma, then the variant-13 mix). Ids are sorted by (hash, id).
// ----------------------------------------------------------------------------
__device__ __forceinline__ uint64_t splitmix_at(uint64_t seed, uint64_t ctr) {
    uint64_t z = seed + (ctr + 1ull) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// perm[i] = the i-th id (0-based, relative to id0) of `count` ids in random order.
// Every thread of the workgroup must call it; ends with a barrier.
__device__ void build_order(uint16_t* perm, uint64_t seed, int64_t row, int tag, int64_t id0,
                            int count, unsigned char* scratch) {
    const uint64_t ctr0 = ((uint64_t)(row * 2 + tag) << 32) + (uint64_t)id0;
    if (count <= 64) {
        if (wave_id() == 0) {
            const int lane = lane_id();
            const uint64_t h = lane < count ? splitmix_at(seed, ctr0 + lane) : ~0ull;
            const uint32_t hl = (uint32_t)h, hh = (uint32_t)(h >> 32);
            int rank = 0;
            for (int i = 0; i < count; ++i) {
                const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(hh, i) << 32) |
                                   (uint32_t)__builtin_amdgcn_readlane(hl, i);
                rank += (o < h) || (o == h && i < lane);
            }
            if (lane < count) perm[rank] = (uint16_t)lane;
        }
    } else {
        const int p2 = (int)next_pow2(count);
        uint64_t* hk = reinterpret_cast<uint64_t*>(scratch);
        uint32_t* hid = reinterpret_cast<uint32_t*>(scratch + (size_t)p2 * 8);
        for (int i = threadIdx.x; i < p2; i += kWG) {
            hk[i] = i < count ? splitmix_at(seed, ctr0 + (uint64_t)i) : ~0ull;
            hid[i] = (uint32_t)i;
        }
        __syncthreads();
        for (int size = 2; size <= p2; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int i = threadIdx.x; i < p2; i += kWG) {
                    const int j = i ^ stride;
                    if (j > i) {
                        const uint64_t a = hk[i], b = hk[j];
                        const uint32_t ia = hid[i], ib = hid[j];
                        const bool a_gt = a > b || (a == b && ia > ib);
                        const bool up = (i & size) == 0;
                        if (a_gt == up) {
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
        for (int i = threadIdx.x; i < count; i += kWG) perm[i] = (uint16_t)hid[i];
    }
    __syncthreads();
}

// ----------------------------------------------------------------------------
// Append the survivors of one tile (one predicate per slot and lane) to the
// candidate buffer at len: wave counts from the ballot masks, a prefix over the
// 4 waves through LDS (one barrier), then each survivor's slot from mbcnt.
// `put(slot, pos)` stores slot's element at buffer position pos. Returns the
// number appended by the whole workgroup (uniform).
// ----------------------------------------------------------------------------
template <int NS, class Put>
__device__ __forceinline__ uint32_t append_masked(const uint64_t (&masks)[NS], const bool (&pred)[NS],
                                                  uint32_t len, uint32_t* cnt, uint32_t& par, Put&& put) {
    uint32_t c = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) c += (uint32_t)__popcll(masks[s]);
    const int wave = wave_id();
    if (lane_id() == 0) cnt[par * kWaves + wave] = c;
    __syncthreads();
    const u32x4 cc = *reinterpret_cast<const u32x4*>(cnt + par * kWaves);
    par ^= 1u;
    const uint32_t base = (wave > 0 ? cc.x : 0u) + (wave > 1 ? cc.y : 0u) + (wave > 2 ? cc.z : 0u);
    const uint32_t total = uniform(cc.x + cc.y + cc.z + cc.w);
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

// ----------------------------------------------------------------------------
// RadixSelectTopK in LDS.
// ----------------------------------------------------------------------------
struct SelectScratch {
    uint32_t* hist;  // 2 sets x kWaves x 256
    uint32_t* pcnt;  // 2 x kWaves x 2
    uint32_t hset;   // set whose private histograms are all zero
};

// Zero both histogram sets of this wave (call at the start of a workgroup's work,
// after a barrier that ends every earlier reader).
__device__ __forceinline__ void zero_hist(SelectScratch& sc) {
    const int wave = wave_id(), lane = lane_id();
    for (int set = 0; set < 2; ++set) {
        u32x4* h = reinterpret_cast<u32x4*>(sc.hist + (set * kWaves + wave) * 256);
        h[lane] = u32x4{0u, 0u, 0u, 0u};
    }
    sc.hset = 0;
}

// Inclusive suffix sum over the 64 lanes (lane l gets sum of lanes >= l).
__device__ __forceinline__ uint32_t wave_suffix_sum(uint32_t v) {
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_down(v, d, 64);
        if (lane + d < 64) v += o;
    }
    return v;
}

// Stable in-place partition of keys/idx[0, n): keep every key > kth and the
// first `need` keys == kth in buffer order, packed into [0, k). Rounds of
// kWG*R entries: every wave reads its 64*R entries into registers, publishes
// (greater, tied) counts, one barrier, then writes; a destination never lies
// beyond its source, so no round overwrites an entry not yet read.
template <class KeyT, int R = 8>
__device__ void partition_keep(KeyT* keys, uint32_t* idx, uint32_t n, uint32_t kth, uint32_t need,
                               uint32_t* pcnt) {
    const int lane = lane_id(), wave = wave_id();
    uint32_t sel_run = 0, tie_run = 0, par = 0;
    for (uint32_t base = 0; base < n; base += kWG * R) {
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
            gm[r] = __ballot(v && kk[r] > kth);
            tm[r] = __ballot(v && kk[r] == kth);
            g += (uint32_t)__popcll(gm[r]);
            t += (uint32_t)__popcll(tm[r]);
        }
        if (lane == 0) {
            pcnt[(par * kWaves + wave) * 2 + 0] = g;
            pcnt[(par * kWaves + wave) * 2 + 1] = t;
        }
        __syncthreads();
        uint32_t sel_before = sel_run, tie_before = tie_run, sel_round = 0, tie_round = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t gw = pcnt[(par * kWaves + w) * 2 + 0];
            const uint32_t tw = pcnt[(par * kWaves + w) * 2 + 1];
            const uint32_t ties_prior = tie_run + tie_round;
            const uint32_t room = need > ties_prior ? need - ties_prior : 0u;
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
            const uint64_t lt = lanes_below(tm[r]);
            const bool is_tie = (tm[r] >> lane) & 1ull;
            const bool is_gt = (gm[r] >> lane) & 1ull;
            const bool sel = is_gt || (is_tie && tb + (uint32_t)lt < need);
            const uint64_t sm = __ballot(sel);
            if (sel) {
                const uint32_t dst = sb + lanes_below(sm);
                keys[dst] = (KeyT)kk[r];
                idx[dst] = ii[r];
            }
            tb += (uint32_t)__popcll(tm[r]);
            sb += (uint32_t)__popcll(sm);
        }
        sel_run += uniform(sel_round);
        tie_run += uniform(tie_round);
    }
}

// Keep the k largest of keys/idx[0, n) (n > k) in [0, k); return the k-th key.
// MSD select over 8-bit digits: each pass histograms, into the wave's private
// copy, the digit of every key that matches the prefix fixed so far; after one
// barrier every wave sums the 4 copies and walks the bins from the top to the
// one holding the rank-th largest (the walk is a 64-lane suffix scan plus a
// 4-bin step). The histogram set alternates between passes; each wave clears
// its own copy of the set it is not using once every reader has passed the
// barrier, so a pass costs one barrier.
template <class D>
__device__ uint32_t radix_select(typename D::Key* keys, uint32_t* idx, uint32_t n, uint32_t k,
                                 SelectScratch& sc) {
    const int lane = lane_id(), wave = wave_id();
    __syncthreads();  // every append / earlier partition is visible
    uint32_t prefix = 0, pmask = 0, rank = k;
#pragma unroll
    for (int shift = D::kBits - 8; shift >= 0; shift -= 8) {
        uint32_t* hw = sc.hist + (sc.hset * kWaves + wave) * 256;
        for (uint32_t i = threadIdx.x; i < n; i += kWG) {
            const uint32_t key = keys[i];
            if ((key & pmask) == prefix) atomicAdd(&hw[(key >> shift) & 0xFFu], 1u);
        }
        __syncthreads();
        // clear this wave's copy in the other set: its readers (the previous
        // pass's digit walk) have all passed the barrier above
        reinterpret_cast<u32x4*>(sc.hist + ((sc.hset ^ 1u) * kWaves + wave) * 256)[lane] =
            u32x4{0u, 0u, 0u, 0u};
        const u32x4* hs = reinterpret_cast<const u32x4*>(sc.hist + sc.hset * kWaves * 256);
        u32x4 c = hs[lane];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) c += hs[w * 64 + lane];
        const uint32_t s = c.x + c.y + c.z + c.w;  // digits 4*lane .. 4*lane+3
        const uint32_t incl = wave_suffix_sum(s);
        const uint64_t ge = __ballot(incl >= rank);
        const int L = 63 - __clzll((long long)ge);
        uint32_t above = uniform(__builtin_amdgcn_readlane(incl - s, L));
        const uint32_t c3 = uniform(__builtin_amdgcn_readlane(c.w, L));
        const uint32_t c2 = uniform(__builtin_amdgcn_readlane(c.z, L));
        const uint32_t c1 = uniform(__builtin_amdgcn_readlane(c.y, L));
        uint32_t d;
        if (above + c3 >= rank) {
            d = 4u * L + 3u;
        } else if (above + c3 + c2 >= rank) {
            above += c3;
            d = 4u * L + 2u;
        } else if (above + c3 + c2 + c1 >= rank) {
            above += c3 + c2;
            d = 4u * L + 1u;
        } else {
            above += c3 + c2 + c1;
            d = 4u * L;
        }
        rank -= above;
        prefix |= d << shift;
        pmask |= 0xFFu << shift;
        sc.hset ^= 1u;
    }
    partition_keep<typename D::Key>(keys, idx, n, prefix, rank, sc.pcnt);
    return prefix;
}

}  // namespace ds
