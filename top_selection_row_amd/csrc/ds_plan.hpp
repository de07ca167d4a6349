// ds_plan.hpp -- shapes, limits and memory layouts of the DeepSelect library.
//
// Plain C++ (no HIP): used by the host side of the library to validate calls,
// pick the split factor, size LDS and the workspace, and by the kernels to find
// their LDS arrays. Everything here is integer bookkeeping.
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

constexpr int kWG = 256;                 // lanes per workgroup (4 waves of 64)
constexpr int kWaves = kWG / 64;
constexpr int kTileBytes = kWG * 16;     // one 16-byte load per lane
constexpr int64_t kPermMax = 8192;       // blocks per part kept in the LDS block order
constexpr int64_t kMaxSplit = 1024;      // parts per row
constexpr size_t kLdsLimit = 160 * 1024; // gfx950 LDS per workgroup
constexpr int64_t kPartBytesMax = (int64_t)1 << 31;  // 32-bit buffer offsets per part

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
        const int64_t e = std::min(b1 * B, n) - b0 * B;
        best = std::min(best, e);
    }
    return best;
}

// Largest part in bytes and in blocks.
inline int64_t max_part_blocks(int64_t m, int64_t S) { return ceil_div(m, S); }

// Dynamic LDS layout of one workgroup (byte offsets from the start of LDS).
struct Layout {
    uint32_t keys;   // cap candidate keys (uint32 for f32, uint16 for bf16)
    uint32_t idx;    // cap candidate column indices (uint32)
    uint32_t hist;   // 2 sets x kWaves private 256-bin histograms (uint32)
    uint32_t cnt;    // 2 x kWaves per-wave survivor counts (block loop)
    uint32_t pcnt;   // 2 x kWaves x 2 per-wave counts (partition)
    uint32_t perm;   // block order (uint16 per block)
    uint32_t misc;   // 16 uint32 of broadcast scratch
    uint32_t total;  // bytes
    int32_t cap;     // candidate buffer capacity in entries
};

// Candidate capacity: the buffer holds < k+B2 entries before a block and gains
// at most one block, so k+B+B2-1 entries suffice; the merge of split rows adds
// blocks of k entries, so it needs 2k+B2-1.
inline int64_t capacity(int64_t k, int64_t B, int64_t B2, int64_t S) {
    int64_t cap = k + B + B2 - 1;
    if (S > 1) cap = std::max(cap, 2 * k + B2 - 1);
    return cap;
}

inline Layout make_layout(int dtype, int64_t n, int64_t k, int64_t B, int64_t B2, int64_t S) {
    Layout L{};
    const int64_t cap = capacity(k, B, B2, S);
    const int64_t m = ceil_div(n, B);
    const int64_t ms = max_part_blocks(m, S);
    const int64_t order_n = std::max<int64_t>(ms, S > 1 ? S : 1);
    size_t off = 0;
    L.keys = 0;
    off = align_up((size_t)cap * elem_bytes(dtype), 16);
    L.idx = (uint32_t)off;
    off = align_up(off + (size_t)cap * 4, 16);
    // The bitonic sort of the block order (more than 64 blocks) uses the
    // candidate arrays as scratch before the scan starts: 8-byte hash + 4-byte id.
    if (order_n > 64) off = std::max(off, align_up((size_t)next_pow2(order_n) * 12, 16));
    L.hist = (uint32_t)off;
    off += 2 * kWaves * 256 * 4;
    L.cnt = (uint32_t)off;
    off += 2 * kWaves * 4;
    L.pcnt = (uint32_t)off;
    off += 2 * kWaves * 2 * 4;
    L.perm = (uint32_t)off;
    off = align_up(off + (size_t)order_n * 2, 16);
    L.misc = (uint32_t)off;
    off += 16 * 4;
    L.total = (uint32_t)align_up(off, 16);
    L.cap = (int32_t)cap;
    return L;
}

// Workspace of split rows (device memory). The arrival counters come first so a
// caller only has to zero the first batch*4 bytes (zeroing all of it is fine).
struct WsLayout {
    size_t arrive, keys, idx, stats, total;
};

inline WsLayout make_ws_layout(int64_t batch, int64_t k, int64_t S) {
    WsLayout w{};
    if (S <= 1) return w;
    size_t off = 0;
    w.arrive = off;
    off = align_up(off + (size_t)batch * 4, 256);
    w.keys = off;
    off = align_up(off + (size_t)batch * S * k * 4, 256);
    w.idx = off;
    off = align_up(off + (size_t)batch * S * k * 4, 256);
    w.stats = off;
    off = align_up(off + (size_t)batch * S * 4 * 8, 256);
    w.total = off;
    return w;
}

}  // namespace ds
