// ds_plan.hpp -- shapes, limits and memory layouts of the DeepSelect library.
//
// Integer bookkeeping shared by the host side (argument checks, split factor,
// LDS and workspace sizes) and the kernels (where their LDS arrays live).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>

// Helpers the kernels also call are marked for both host and device.
#ifdef __HIPCC__
#define DS_HD __host__ __device__
#else
#define DS_HD
#endif

namespace ds {

constexpr int kUnitBytes = 1024;          // one 16-byte load per lane of a wave
constexpr int64_t kPermMax = 8192;        // blocks per part kept in the LDS block order
constexpr int64_t kMaxSplit = 1024;       // parts per row
constexpr size_t kLdsLimit = 160 * 1024;  // gfx950 LDS per workgroup
constexpr int64_t kPartBytesMax = (int64_t)1 << 31;  // 32-bit buffer offsets per part
constexpr int kChunk = 8;                 // candidate entries per thread and select round
constexpr int kRoundsPerGroup = 2;        // select rounds whose entries a thread holds at once
constexpr int kGather = 256;              // radix bins this small are finished by every wave alone
constexpr int kMiscWords = 32;            // [16, 32): four copies of the row's shared cell

DS_HD inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
DS_HD inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
DS_HD inline int64_t next_pow2(int64_t v) {
    int64_t p = 1;
    while (p < v) p <<= 1;
    return p;
}
DS_HD inline int elem_bytes(int dtype) { return dtype == 0 ? 4 : 2; }

// Block range [b0, b1) of part s of S over m blocks.
DS_HD inline int64_t part_begin(int64_t m, int64_t s, int64_t S) { return s * m / S; }

// Smallest element count over the parts of a row split S ways.
inline int64_t min_part_elems(int64_t n, int64_t B, int64_t S) {
    const int64_t m = ceil_div(n, B);
    int64_t best = n;
    for (int64_t s = 0; s < S; ++s) {
        const int64_t b0 = part_begin(m, s, S), b1 = part_begin(m, s + 1, S);
        best = std::min(best, std::min(b1 * B, n) - b0 * B);
    }
    return best;
}

// Dynamic LDS layout of one workgroup (byte offsets from the start of LDS).
struct Layout {
    uint32_t keys;   // cap candidate keys (uint32 for f32, uint16 for bf16), padded to 8 entries,
                     // then 64 junk entries (stores of dropped entries)
    uint32_t idx;    // cap candidate column indices (uint32), the same padding and junk
    uint32_t hist;   // radix histogram: 16 copies of 256 16-bit counters (8 KiB)
    uint32_t fold;   // 256 folded bins (uint32)
    uint32_t gather; // kGather keys of one radix bin (uint32), gathered for a wave-local finish
    uint32_t tot;    // 2 x rounds x waves per-wave totals of the select partition
    uint32_t cnt;    // 2 x waves per-wave counts (block loop)
    uint32_t perm;   // block order (uint16 per block)
    uint32_t misc;   // kMiscWords uint32 of broadcast scratch
    uint32_t ring;   // streaming ring: waves x ring_depth blocks of ring_units KiB (0 if none)
    uint32_t sort;   // sorted output: next_pow2(k) uint64 sort words (0 if not asked for)
    uint32_t pcnt;   // merge: one count per part (0 if none)
    uint32_t total;  // bytes
    int32_t cap;     // candidate buffer capacity in entries
    int32_t junk;    // first junk entry (cap padded to 8)
    int32_t ring_depth;  // blocks per wave in the ring (0: no ring)
    int32_t ring_units;  // KiB per block slot
    int32_t waves;   // waves per workgroup the layout was made for
};

// Candidate capacity: the buffer holds < k+B2 entries before a block and a
// block adds at most its length, so k + blk + B2 - 1 entries suffice.
inline int64_t capacity(int64_t k, int64_t blk, int64_t B2) { return k + blk + B2 - 1; }

// order_n: ids in the random order (blocks of the largest part, or parts).
// key_bytes 0: packed entries (a 16-bit key and a 16-bit part-local column in
// one 32-bit word), with no column array.
inline Layout make_layout_raw(int key_bytes, int64_t cap, int64_t order_n, int waves) {
    Layout L{};
    const int64_t capp = ceil_div(cap, kChunk) * kChunk;
    const int64_t entries = capp + 64;
    const bool packed = key_bytes == 0;
    size_t off = 0;
    L.keys = 0;
    off = align_up((size_t)entries * (packed ? 4 : key_bytes), 16);
    L.idx = (uint32_t)off;
    if (!packed) off = align_up(off + (size_t)entries * 4, 16);
    // Building the block order uses the candidate arrays as scratch before the
    // scan starts: an 8-byte hash and a 4-byte rank or id per entry.
    off = std::max(off, align_up((size_t)next_pow2(std::max<int64_t>(order_n, 1)) * 12, 16));
    L.hist = (uint32_t)off;
    off += (size_t)16 * 128 * 4;
    L.fold = (uint32_t)off;
    off += 256 * 4;
    L.gather = (uint32_t)off;
    off += kGather * 4;
    L.tot = (uint32_t)off;
    off += align_up((size_t)2 * kRoundsPerGroup * waves * 4, 16);
    L.cnt = (uint32_t)off;
    off += align_up((size_t)2 * waves * 4, 16);
    L.perm = (uint32_t)off;
    off = align_up(off + (size_t)order_n * 2, 16);
    L.misc = (uint32_t)off;
    off += kMiscWords * 4;
    L.total = (uint32_t)align_up(off, 16);
    L.cap = (int32_t)cap;
    L.junk = (int32_t)capp;
    L.waves = waves;
    return L;
}

// Layout of the streaming kernel: a part of ceil(m/S) blocks.
inline Layout make_layout(int dtype, int64_t n, int64_t k, int64_t B, int64_t B2, int64_t S, int waves,
                          bool packed = false) {
    const int64_t m = ceil_div(n, B);
    return make_layout_raw(packed ? 0 : elem_bytes(dtype), capacity(k, std::min<int64_t>(B, n), B2), ceil_div(m, S),
                           waves);
}

// bfloat16 parts of at most 65536 elements keep each candidate as one 32-bit
// word, key << 16 | part-local column.
inline bool packed_parts(int dtype, int64_t n, int64_t B, int64_t S) {
    const int64_t m = ceil_div(n, B);
    return dtype == 1 && ceil_div(m, S) * B <= 65536;
}

// Add a streaming ring to a layout: every wave gets `depth` slots of `units`
// KiB, depth as large as LDS allows up to kRingMax (and no more than the steps
// of a part). Leaves the layout without a ring when fewer than 2 slots fit.
// Two slots (one block landing while the wave works on the other) measured as
// fast as or faster than three or four on every workload here.
constexpr int kRingMax = 2;
inline Layout with_ring(Layout L, int64_t steps, int units, size_t lds_limit) {
    const size_t base = align_up(L.total, 16);
    const size_t per = (size_t)L.waves * units * kUnitBytes;
    int64_t depth = base < lds_limit ? (int64_t)((lds_limit - base) / per) : 0;
    depth = std::min<int64_t>({depth, (int64_t)kRingMax, std::max<int64_t>(steps, 1)});
    if (depth < 2 && !(depth == 1 && steps <= 1)) return L;
    L.ring = (uint32_t)base;
    L.ring_depth = (int32_t)depth;
    L.ring_units = units;
    L.total = (uint32_t)(base + per * depth);
    return L;
}

// Room for sorting a row's k results before they are written: next_pow2(k)
// 64-bit words (key << 32 | ~column).
inline Layout with_sort(Layout L, int64_t k) {
    const size_t base = align_up(L.total, 16);
    L.sort = (uint32_t)base;
    L.total = (uint32_t)(base + (size_t)next_pow2(k) * 8);
    return L;
}

// Layout of the merge kernel of split rows: S blocks of k candidates.
// The merge also keeps one count per part (uint32, in `pcnt`).
inline Layout make_merge_layout(int dtype, int64_t k, int64_t B2, int64_t S, int waves) {
    Layout L = make_layout_raw(elem_bytes(dtype), capacity(k, k, B2), S, waves);
    L.pcnt = (uint32_t)align_up(L.total, 16);
    L.total = (uint32_t)align_up(L.pcnt + (size_t)S * 4, 16);
    return L;
}

// Workspace of split rows (device memory): every part's k (key, column) pairs
// and its four statistics. The merge kernel reads it after the part kernel.
struct WsLayout {
    size_t keys, idx, stats, cnt, tkey, tmax, share, total;
};

// Shared-threshold cells: one uint64 per row, each on a 128-byte line of its
// own (the rows' parts update and read their cells while other rows do the
// same). A workspace the library owns, and the static scratch, keep kCells of
// them reserved at their start, whatever the shape of the call.
constexpr int64_t kCells = 1024;
constexpr int64_t kCellWords = 16;  // uint64 words from one row's cell to the next
constexpr int64_t kArriveWord = 8;  // the word of a row's cell counting its ended parts

// The shared-threshold cells come first: max(batch, cells) of them, so with
// cells = kCells the first kCells sit at the same place for every call and no
// other array of any call overlaps them.
inline WsLayout make_ws_layout(int64_t batch, int64_t k, int64_t S, int64_t cells = 0) {
    WsLayout w{};
    if (S <= 1) return w;
    size_t off = 0;
    w.share = off;  // each row's shared threshold key + 1 (uint64; the merge leaves it 0)
    off = align_up(off + (size_t)std::max(batch, cells) * kCellWords * 8, 256);
    w.keys = off;
    off = align_up(off + (size_t)batch * S * k * 4, 256);
    w.idx = off;
    off = align_up(off + (size_t)batch * S * k * 4, 256);
    w.stats = off;
    off = align_up(off + (size_t)batch * S * 4 * 8, 256);
    w.cnt = off;  // each part's number of results (uint32)
    off = align_up(off + (size_t)batch * S * 4, 256);
    w.tkey = off;  // each part's k-th key when it has k results, else 0 (uint32)
    off = align_up(off + (size_t)batch * S * 4, 256);
    w.tmax = off;  // each part's largest result key, 0 without results (uint32)
    off = align_up(off + (size_t)batch * S * 4, 256);
    w.total = off;
    return w;
}

}  // namespace ds
