// deepselect.hip -- MI355X (gfx950) DeepSelect batched row-wise top-k and its C ABI.
//
// DeepSelect (DeepSelect deep-dive, PFCCLab/DeepSelect, section "算法"): each row
// is read once, in B-element blocks taken in a random order independent of the
// data. Elements above the threshold T go to an on-chip candidate buffer; when
// the buffer reaches k + B2 entries a radix select keeps its k largest and T
// becomes the k-th. A final select returns k. Before the first compaction every
// element is admitted (the page says so right after the pseudo-code).
//
// Mapping on gfx950
//   * one 256-lane workgroup per (row, part); the candidate buffer (keys + column
//     indices), the radix histograms and the block order live in LDS;
//   * a block is streamed as 4 KiB tiles, one 16-byte buffer load per lane, kept
//     P tiles ahead in a register ring (the block order is known up front, so
//     loads never wait on the filter); lanes past the end of a block get an
//     out-of-range buffer offset, which returns zero and touches no memory;
//   * the filter compares raw bits against the threshold (signed compare when
//     T >= +0, unsigned "less than" when T < 0, both exact under the key order)
//     and compacts survivors with 64-bit ballot masks, mbcnt ranks and one
//     4-wave prefix through LDS;
//   * split rows (the deep-dive's "实现" section, last paragraph: a row cut into
//     parts whose top-k go to one reducer): each part writes its k results to a
//     device workspace, publishes them with an agent-scope release and an
//     arrival counter, and the last part to arrive runs DeepSelect once more
//     over the parts' results (one block per part) and writes the row.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <map>
#include <mutex>
#include <utility>

#include "../../include/deepselect.h"
#include "ds_device.hpp"
#include "ds_plan.hpp"

namespace ds {

constexpr uint32_t kOob = 0x80000000u;  // buffer offset past every part (parts < 2 GiB)
constexpr uint32_t kRsrcWord3 = 0x00020000u;

struct Params {
    const void* x;
    void* out_vals;
    int32_t* out_idx;
    uint64_t* stats;
    uint32_t* ws_arrive;
    uint32_t* ws_keys;
    uint32_t* ws_idx;
    uint64_t* ws_stats;
    int64_t batch, n, row_stride, m;
    uint64_t seed;
    int32_t k, B, B2, split, tpb;
    Layout L;
};

struct RunState {
    uint32_t len = 0;      // candidate entries
    bool tset = false;     // threshold set (a compaction happened)
    uint32_t tkey = 0;     // threshold key
    uint64_t W = 0, A = 0, R = 0, maxlen = 0;
    uint32_t par = 0;      // count-buffer parity
};

template <class D>
struct Lds {
    typename D::Key* keys;
    uint32_t* idx;
    uint32_t* cnt;
    uint16_t* perm;
    uint32_t* misc;
    SelectScratch sc;
    unsigned char* base;
};

template <class D>
__device__ __forceinline__ Lds<D> lds_of(unsigned char* smem, const Layout& L) {
    Lds<D> s;
    s.base = smem;
    s.keys = reinterpret_cast<typename D::Key*>(smem + L.keys);
    s.idx = reinterpret_cast<uint32_t*>(smem + L.idx);
    s.cnt = reinterpret_cast<uint32_t*>(smem + L.cnt);
    s.perm = reinterpret_cast<uint16_t*>(smem + L.perm);
    s.misc = reinterpret_cast<uint32_t*>(smem + L.misc);
    s.sc.hist = reinterpret_cast<uint32_t*>(smem + L.hist);
    s.sc.pcnt = reinterpret_cast<uint32_t*>(smem + L.pcnt);
    s.sc.hset = 0;
    return s;
}

// RadixSelectTopK kept out of line so one copy serves every unrolled ring
// slot. Arguments and result travel by value (k-th key in the low word, the
// clean histogram set in the high word) so nothing lives in scratch memory.
template <class D>
__device__ __noinline__ uint64_t compact_call(typename D::Key* keys, uint32_t* idx, uint32_t* hist,
                                              uint32_t* pcnt, uint32_t n, uint32_t k, uint32_t hset) {
    SelectScratch sc{hist, pcnt, hset};
    const uint32_t kth = radix_select<D>(keys, idx, n, k, sc);
    return ((uint64_t)sc.hset << 32) | kth;
}

// Compaction after a block: RadixSelectTopK(buffer, k), T = k-th key.
template <class D>
__device__ __forceinline__ void maybe_compact(Lds<D>& s, RunState& st, uint32_t k, uint32_t B2) {
    st.maxlen = st.len > st.maxlen ? st.len : st.maxlen;
    if (st.len >= k + B2) {
        st.W += st.len;
        st.R += 1;
        const uint64_t r = compact_call<D>(s.keys, s.idx, s.sc.hist, s.sc.pcnt, st.len, k, s.sc.hset);
        st.tkey = (uint32_t)r;
        s.sc.hset = (uint32_t)(r >> 32);
        st.tset = true;
        st.len = k;
    }
}

// ---------------------------------------------------------------------------
// Raw row source: tiles of 256 lanes x 16 bytes.
// ---------------------------------------------------------------------------
template <class D, bool kVec>
struct RowTiles {
    static constexpr int kPer = D::kPerLoad;           // elements per lane per tile
    static constexpr int kTE = kWG * kPer;              // elements per tile
    using Reg = u32x4;                                  // kVec: one 16-byte load
    struct Ring {
        u32x4 v[kVec ? 1 : (kPer + 3) / 4];
    };
};

template <class D, bool kVec>
__device__ __forceinline__ void load_tile(typename RowTiles<D, kVec>::Ring& r, __amdgpu_buffer_rsrc_t rsrc,
                                          int64_t elem_off, int32_t tv) {
    constexpr int kPer = D::kPerLoad;
    const int lane = threadIdx.x;
    if constexpr (kVec) {
        const bool ok = (lane + 1) * kPer <= tv;
        const uint32_t off = ok ? (uint32_t)((elem_off + (int64_t)lane * kPer) * D::kBytes) : kOob;
        r.v[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
    } else {
#pragma unroll
        for (int s = 0; s < kPer; ++s) {
            const int e = s * kWG + lane;
            const uint32_t off = e < tv ? (uint32_t)((elem_off + e) * D::kBytes) : kOob;
            uint32_t val;
            if constexpr (D::kBytes == 4)
                val = __builtin_amdgcn_raw_buffer_load_b32(rsrc, off, 0, 0);
            else
                val = __builtin_amdgcn_raw_buffer_load_b16(rsrc, off, 0, 0);
            r.v[s / 4][s % 4] = val;
        }
    }
}

// Raw pattern of slot s of this lane's part of a tile, and its element offset
// inside the tile.
template <class D, bool kVec>
__device__ __forceinline__ uint32_t slot_raw(const typename RowTiles<D, kVec>::Ring& r, int s) {
    if constexpr (kVec && D::kBytes == 2) {
        const uint32_t w = r.v[0][s >> 1];
        return (s & 1) ? (w >> 16) : (w & 0xFFFFu);
    } else {
        return r.v[s / 4][s % 4];
    }
}
template <class D, bool kVec>
__device__ __forceinline__ int slot_elem(int s) {
    if constexpr (kVec)
        return (int)threadIdx.x * D::kPerLoad + s;
    else
        return s * kWG + (int)threadIdx.x;
}

// Filter predicate of slot s against threshold constants (T set).
// f32: neg ? raw < traw (unsigned) : (int)raw > (int)traw.
// bf16 (raw in the top half of a 32-bit word): neg ? w < thr : (int)w > (int)thr
// with thr = traw<<16 (neg) or traw<<16 | 0xFFFF.
template <class D, bool kVec>
__device__ __forceinline__ bool slot_pass(const typename RowTiles<D, kVec>::Ring& r, int s, bool neg,
                                          uint32_t thr) {
    if constexpr (D::kBytes == 4) {
        const uint32_t u = r.v[s / 4][s % 4];
        return neg ? (u < thr) : ((int32_t)u > (int32_t)thr);
    } else {
        uint32_t w;
        if constexpr (kVec) {
            const uint32_t d = r.v[0][s >> 1];
            w = (s & 1) ? d : (d << 16);
        } else {
            w = r.v[s / 4][s % 4] << 16;
        }
        return neg ? (w < thr) : ((int32_t)w > (int32_t)thr);
    }
}

template <class D>
__device__ __forceinline__ void threshold_consts(const RunState& st, bool& neg, uint32_t& thr) {
    if constexpr (D::kBytes == 4) {
        neg = st.tkey < 0x80000000u;
        thr = D::raw(st.tkey);
    } else {
        neg = st.tkey < 0x8000u;
        const uint32_t t = D::raw(st.tkey) << 16;
        thr = neg ? t : (t | 0xFFFFu);
    }
}

// Process one tile: admit-all before the first compaction, else filter.
template <class D, bool kVec>
__device__ __forceinline__ void process_tile(Lds<D>& s, RunState& st, const typename RowTiles<D, kVec>::Ring& r,
                                             int64_t elem_base, int32_t tv) {
    constexpr int kPer = D::kPerLoad;
    if (tv <= 0) return;
    if (!st.tset) {
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int e = slot_elem<D, kVec>(q);
            if (e < tv) {
                const uint32_t pos = st.len + (uint32_t)e;
                s.keys[pos] = (typename D::Key)D::key(slot_raw<D, kVec>(r, q));
                s.idx[pos] = (uint32_t)(elem_base + e);
            }
        }
        st.len += (uint32_t)tv;
        st.A += (uint32_t)tv;
        return;
    }
    bool neg;
    uint32_t thr;
    threshold_consts<D>(st, neg, thr);
    bool pred[kPer];
    uint64_t masks[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const bool inb = kVec ? true : (slot_elem<D, kVec>(q) < tv);
        // vector tiles: lanes past tv loaded zeros; exclude them explicitly
        const bool valid = kVec ? ((int)threadIdx.x * kPer < tv) : inb;
        pred[q] = valid && slot_pass<D, kVec>(r, q, neg, thr);
        masks[q] = __ballot(pred[q]);
    }
    const uint32_t added = append_masked<kPer>(masks, pred, st.len, s.cnt, st.par, [&](int q, uint32_t pos) {
        s.keys[pos] = (typename D::Key)D::key(slot_raw<D, kVec>(r, q));
        s.idx[pos] = (uint32_t)(elem_base + slot_elem<D, kVec>(q));
    });
    st.len += added;
    st.A += added;
}

// Stream the blocks of one part in the random order in s.perm.
template <class D, bool kVec, int P>
__device__ void stream_part(Lds<D>& s, RunState& st, const Params& p, __amdgpu_buffer_rsrc_t rsrc,
                            int64_t part_elem0, int64_t part_n, int32_t ms) {
    using Ring = typename RowTiles<D, kVec>::Ring;
    constexpr int kTE = RowTiles<D, kVec>::kTE;
    const int32_t tpb = p.tpb;
    const int64_t B = p.B;
    const int32_t ntiles = ms * tpb;
    const uint32_t k = (uint32_t)p.k, B2 = (uint32_t)p.B2;

    // load-side cursor
    int32_t lblk = 0, lsub = 0;
    auto tile_geom = [&](int32_t bi, int32_t sub, int64_t& off, int32_t& tv) {
        if (bi >= ms) {
            off = 0;
            tv = 0;
            return;
        }
        const int64_t b = (int64_t)uniform(s.perm[bi]);
        const int64_t blen = (b * B + B <= part_n) ? B : (part_n - b * B);
        const int64_t rem = blen - (int64_t)sub * kTE;
        tv = (int32_t)(rem < kTE ? (rem > 0 ? rem : 0) : kTE);
        off = b * B + (int64_t)sub * kTE;
    };
    auto advance = [&](int32_t& bi, int32_t& sub) {
        if (++sub == tpb) {
            sub = 0;
            ++bi;
        }
    };

    Ring ring[P];
#pragma unroll
    for (int j = 0; j < P; ++j) {
        int64_t off;
        int32_t tv;
        tile_geom(lblk, lsub, off, tv);
        load_tile<D, kVec>(ring[j], rsrc, off, tv);
        advance(lblk, lsub);
        __builtin_amdgcn_sched_barrier(0);
    }
    int32_t pblk = 0, psub = 0;
    for (int32_t t0 = 0; t0 < ntiles; t0 += P) {
#pragma unroll
        for (int j = 0; j < P; ++j) {
            if (t0 + j < ntiles) {
                int64_t off;
                int32_t tv;
                tile_geom(pblk, psub, off, tv);
                process_tile<D, kVec>(s, st, ring[j], part_elem0 + off, tv);
                if (psub == tpb - 1) maybe_compact<D>(s, st, k, B2);
                advance(pblk, psub);
            }
            int64_t off;
            int32_t tv;
            tile_geom(lblk, lsub, off, tv);
            load_tile<D, kVec>(ring[j], rsrc, off, tv);
            advance(lblk, lsub);
        }
    }
}

// Final RadixSelectTopK (its input length counts in W).
template <class D>
__device__ __forceinline__ void final_select(Lds<D>& s, RunState& st, uint32_t k) {
    st.W += st.len;
    if (st.len > k) {
        st.tkey = radix_select<D>(s.keys, s.idx, st.len, k, s.sc);
        st.len = k;
    }
    __syncthreads();
}

// Merge of split rows: DeepSelect over the parts' results, one block per part.
template <class D>
__device__ void merge_parts(Lds<D>& s, RunState& st, const Params& p, int64_t row) {
    const uint32_t k = (uint32_t)p.k, B2 = (uint32_t)p.B2;
    const int32_t S = p.split;
    build_order(s.perm, p.seed, row, 1, 0, S, s.base);
    for (int32_t i = 0; i < S; ++i) {
        const int64_t part = (int64_t)uniform(s.perm[i]);
        const uint32_t* wk = p.ws_keys + (row * S + part) * (int64_t)k;
        const uint32_t* wi = p.ws_idx + (row * S + part) * (int64_t)k;
        for (uint32_t t0 = 0; t0 < k; t0 += kWG * 4) {
            const uint32_t tv = (k - t0) < (uint32_t)(kWG * 4) ? (k - t0) : (uint32_t)(kWG * 4);
            uint32_t kk[4], ii[4];
            bool inb[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t e = (uint32_t)threadIdx.x * 4u + (uint32_t)q;
                inb[q] = e < tv;
                kk[q] = inb[q] ? __builtin_nontemporal_load(wk + t0 + e) : 0u;
                ii[q] = inb[q] ? __builtin_nontemporal_load(wi + t0 + e) : 0u;
            }
            if (!st.tset) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (inb[q]) {
                        const uint32_t pos = st.len + (uint32_t)threadIdx.x * 4u + (uint32_t)q;
                        s.keys[pos] = (typename D::Key)kk[q];
                        s.idx[pos] = ii[q];
                    }
                }
                st.len += tv;
                st.A += tv;
            } else {
                bool pred[4];
                uint64_t masks[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    pred[q] = inb[q] && kk[q] > st.tkey;
                    masks[q] = __ballot(pred[q]);
                }
                const uint32_t added = append_masked<4>(masks, pred, st.len, s.cnt, st.par,
                                                        [&](int q, uint32_t pos) {
                                                            s.keys[pos] = (typename D::Key)kk[q];
                                                            s.idx[pos] = ii[q];
                                                        });
                st.len += added;
                st.A += added;
            }
        }
        maybe_compact<D>(s, st, k, B2);
    }
    final_select<D>(s, st, k);
}

template <class D>
__device__ __forceinline__ void write_row(Lds<D>& s, const RunState& st, const Params& p, int64_t row,
                                          uint64_t W, uint64_t A, uint64_t R, uint64_t maxlen) {
    const int64_t k = p.k;
    for (int64_t j = threadIdx.x; j < k; j += kWG) {
        const uint32_t key = s.keys[j];
        if constexpr (D::kBytes == 4)
            reinterpret_cast<uint32_t*>(p.out_vals)[row * k + j] = D::raw(key);
        else
            reinterpret_cast<uint16_t*>(p.out_vals)[row * k + j] = (uint16_t)D::raw(key);
        p.out_idx[row * k + j] = (int32_t)s.idx[j];
    }
    if (p.stats && threadIdx.x == 0) {
        uint64_t* o = p.stats + row * DS_STATS_PER_ROW;
        o[DS_STAT_W] = W;
        o[DS_STAT_A] = A;
        o[DS_STAT_R] = R;
        o[DS_STAT_MAX_LEN] = maxlen;
    }
}

template <class D, bool kVec, int P>
__global__ __launch_bounds__(kWG) void deepselect_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    Lds<D> s = lds_of<D>(smem, p.L);
    const int64_t items = p.batch * (int64_t)p.split;
    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const int64_t row = item / p.split;
        const int32_t part = (int32_t)(item % p.split);
        __syncthreads();  // LDS free from the previous item
        zero_hist(s.sc);

        const int64_t b0 = part_begin(p.m, part, p.split), b1 = part_begin(p.m, part + 1, p.split);
        const int32_t ms = (int32_t)(b1 - b0);
        const int64_t part_elem0 = b0 * (int64_t)p.B;
        const int64_t part_n = ((b1 * (int64_t)p.B < p.n) ? b1 * (int64_t)p.B : p.n) - part_elem0;
        const unsigned char* rowp = reinterpret_cast<const unsigned char*>(p.x) +
                                    (row * p.row_stride + part_elem0) * D::kBytes;
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<unsigned char*>(rowp), (short)0, (int)(part_n * D::kBytes), (int)kRsrcWord3);

        build_order(s.perm, p.seed, row, 0, b0, ms, s.base);
        RunState st;
        stream_part<D, kVec, P>(s, st, p, rsrc, part_elem0, part_n, ms);
        final_select<D>(s, st, (uint32_t)p.k);

        if (p.split == 1) {
            write_row<D>(s, st, p, row, st.W, st.A, st.R, st.maxlen);
            continue;
        }
        // publish this part's k results and statistics
        const int64_t slot = row * p.split + part;
        for (int64_t j = threadIdx.x; j < p.k; j += kWG) {
            p.ws_keys[slot * p.k + j] = (uint32_t)s.keys[j];
            p.ws_idx[slot * p.k + j] = s.idx[j];
        }
        if (threadIdx.x == 0) {
            uint64_t* o = p.ws_stats + slot * DS_STATS_PER_ROW;
            o[DS_STAT_W] = st.W;
            o[DS_STAT_A] = st.A;
            o[DS_STAT_R] = st.R;
            o[DS_STAT_MAX_LEN] = st.maxlen;
        }
        __threadfence();  // release: this thread's stores are visible device-wide
        __syncthreads();
        if (threadIdx.x == 0) {
            const uint32_t old = atomicAdd(p.ws_arrive + row, 1u);
            s.misc[0] = (old == (uint32_t)p.split - 1u) ? 1u : 0u;
        }
        __syncthreads();
        if (s.misc[0] == 0u) continue;
        __threadfence();  // acquire: the other parts' stores are visible here
        if (threadIdx.x == 0) p.ws_arrive[row] = 0u;  // ready for the next call

        uint64_t W = 0, A = 0, R = 0, maxlen = 0;
        for (int32_t q = 0; q < p.split; ++q) {
            const uint64_t* o = p.ws_stats + (row * p.split + q) * DS_STATS_PER_ROW;
            W += __builtin_nontemporal_load(o + DS_STAT_W);
            A += __builtin_nontemporal_load(o + DS_STAT_A);
            R += __builtin_nontemporal_load(o + DS_STAT_R);
            const uint64_t ml = __builtin_nontemporal_load(o + DS_STAT_MAX_LEN);
            maxlen = ml > maxlen ? ml : maxlen;
        }
        __syncthreads();  // everyone is done with the part's buffer
        RunState mst;
        merge_parts<D>(s, mst, p, row);
        write_row<D>(s, mst, p, row, W + mst.W, A + mst.A, R + mst.R,
                     mst.maxlen > maxlen ? mst.maxlen : maxlen);
    }
}

__global__ void zero_u32_kernel(uint32_t* p, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------

static int validate_shape(int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k, int32_t B,
                          int32_t B2) {
    if (dtype != DS_F32 && dtype != DS_BF16) return DS_ERR_DTYPE;
    if (batch < 0 || n < 1 || n >= ((int64_t)1 << 31) || row_stride < n) return DS_ERR_SHAPE;
    if (k < 1 || k > n) return DS_ERR_K;
    if (B < 1 || B2 < 1) return DS_ERR_BLOCK;
    return DS_OK;
}

static int64_t split_lower_bound(int dtype, int64_t n, int64_t B) {
    const int64_t m = ceil_div(n, B);
    int64_t lo = ceil_div(m, kPermMax);
    const int64_t bytes = n * elem_bytes(dtype);
    lo = std::max<int64_t>(lo, ceil_div(bytes + B * elem_bytes(dtype), kPartBytesMax));
    return std::max<int64_t>(lo, 1);
}

static bool split_ok(int64_t n, int64_t k, int64_t B, int64_t S) {
    const int64_t m = ceil_div(n, B);
    if (S < 1 || S > m || S > kMaxSplit) return false;
    return S == 1 || min_part_elems(n, B, S) >= k;
}

static int lds_check(int dtype, int64_t n, int64_t k, int64_t B, int64_t B2, int64_t S) {
    if ((int64_t)k + B + B2 > ((int64_t)1 << 30)) return DS_ERR_UNSUPPORTED;
    const Layout L = make_layout(dtype, n, k, B, B2, S);
    return L.total <= kLdsLimit ? DS_OK : DS_ERR_UNSUPPORTED;
}

static int plan_split(int dtype, int64_t batch, int64_t n, int32_t k, int32_t B, int32_t B2, int32_t num_cus) {
    const int64_t lo = split_lower_bound(dtype, n, B);
    int64_t S = 1;
    if (batch > 0 && batch < num_cus) S = ceil_div(num_cus, batch);
    const double bal = std::floor(std::sqrt((double)n * elem_bytes(dtype) / (8.0 * (double)k)));
    S = std::min<int64_t>(S, std::max<int64_t>(1, (int64_t)bal));
    S = std::max<int64_t>(S, lo);
    while (S > lo && (!split_ok(n, k, B, S) || lds_check(dtype, n, k, B, B2, S) != DS_OK)) --S;
    if (!split_ok(n, k, B, S)) return DS_ERR_UNSUPPORTED;
    if (lds_check(dtype, n, k, B, B2, S) != DS_OK) return DS_ERR_UNSUPPORTED;
    return (int)S;
}

struct DevInfo {
    int cus = 0;
    int lds = 0;
};

static std::mutex g_mu;
static std::map<int, DevInfo> g_dev;
struct WsBuf {
    void* ptr = nullptr;
    size_t bytes = 0;
};
static std::map<std::pair<int, void*>, WsBuf> g_ws;

static int device_info(int dev, DevInfo& out) {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_dev.find(dev);
    if (it != g_dev.end()) {
        out = it->second;
        return DS_OK;
    }
    DevInfo d;
    if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return DS_ERR_HIP;
    if (hipDeviceGetAttribute(&d.lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
        return DS_ERR_HIP;
    g_dev[dev] = d;
    out = d;
    return DS_OK;
}

static int library_workspace(int dev, hipStream_t stream, size_t bytes, size_t zero_bytes, void** out) {
    std::lock_guard<std::mutex> lk(g_mu);
    WsBuf& w = g_ws[{dev, (void*)stream}];
    if (w.bytes < bytes) {
        if (w.ptr) {
            if (hipStreamSynchronize(stream) != hipSuccess) return DS_ERR_HIP;
            if (hipFree(w.ptr) != hipSuccess) return DS_ERR_HIP;
            w.ptr = nullptr;
            w.bytes = 0;
        }
        void* ptr = nullptr;
        if (hipMalloc(&ptr, bytes) != hipSuccess) return DS_ERR_HIP;
        const int64_t words = (int64_t)(zero_bytes / 4);
        const int grid = (int)std::min<int64_t>(std::max<int64_t>(ceil_div(words, 256), 1), 1024);
        hipLaunchKernelGGL(zero_u32_kernel, dim3(grid), dim3(256), 0, stream, (uint32_t*)ptr, words);
        if (hipGetLastError() != hipSuccess) {
            (void)hipFree(ptr);
            return DS_ERR_HIP;
        }
        w.ptr = ptr;
        w.bytes = bytes;
    }
    *out = w.ptr;
    return DS_OK;
}

template <class D, bool kVec, int P>
static int launch(const Params& prm, size_t lds, hipStream_t stream, int64_t items) {
    auto kern = deepselect_kernel<D, kVec, P>;
    if (lds > 64 * 1024) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
            return DS_ERR_HIP;
    }
    const int64_t grid = std::min<int64_t>(items, (int64_t)1 << 22);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kWG), lds, stream, prm);
    return hipGetLastError() == hipSuccess ? DS_OK : DS_ERR_HIP;
}

static int topk_impl(const void* x, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k,
                     int32_t B, int32_t B2, uint64_t seed, void* out_vals, int32_t* out_idx, void* stream,
                     const ds_options_t* opt) {
    int st = validate_shape(dtype, batch, n, row_stride, k, B, B2);
    if (st != DS_OK) return st;
    if (batch == 0) return DS_OK;
    if (!x || !out_vals || !out_idx) return DS_ERR_NULL;
    const int es = elem_bytes(dtype);
    if (((uintptr_t)x % es) != 0) return DS_ERR_SHAPE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DS_ERR_HIP;
    DevInfo di;
    if ((st = device_info(dev, di)) != DS_OK) return st;

    int64_t S = (opt && opt->split > 0) ? opt->split : 0;
    if (S == 0) {
        const int ps = plan_split(dtype, batch, n, k, B, B2, di.cus);
        if (ps < 0) return ps;
        S = ps;
    } else {
        if (!split_ok(n, k, B, S) || S < split_lower_bound(dtype, n, B)) return DS_ERR_BLOCK;
    }
    if ((st = lds_check(dtype, n, k, B, B2, S)) != DS_OK) return st;
    const Layout L = make_layout(dtype, n, k, B, B2, S);
    if ((int64_t)L.total > (int64_t)di.lds) return DS_ERR_UNSUPPORTED;

    Params prm{};
    prm.x = x;
    prm.out_vals = out_vals;
    prm.out_idx = out_idx;
    prm.stats = opt ? opt->stats : nullptr;
    prm.batch = batch;
    prm.n = n;
    prm.row_stride = row_stride;
    prm.m = ceil_div(n, B);
    prm.seed = seed;
    prm.k = k;
    prm.B = B;
    prm.B2 = B2;
    prm.split = (int32_t)S;
    prm.L = L;

    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    if (S > 1) {
        const WsLayout wl = make_ws_layout(batch, k, S);
        void* ws = nullptr;
        if (opt && opt->workspace) {
            if (opt->workspace_bytes < wl.total) return DS_ERR_WORKSPACE;
            ws = opt->workspace;
        } else if ((st = library_workspace(dev, hs, wl.total, wl.keys, &ws)) != DS_OK) {
            return st;
        }
        unsigned char* w = reinterpret_cast<unsigned char*>(ws);
        prm.ws_arrive = reinterpret_cast<uint32_t*>(w + wl.arrive);
        prm.ws_keys = reinterpret_cast<uint32_t*>(w + wl.keys);
        prm.ws_idx = reinterpret_cast<uint32_t*>(w + wl.idx);
        prm.ws_stats = reinterpret_cast<uint64_t*>(w + wl.stats);
    }
    const bool vec = ((uintptr_t)x % 16 == 0) && ((row_stride * es) % 16 == 0) && (((int64_t)B * es) % 16 == 0) &&
                     ((n * es) % 16 == 0);
    const int te = kWG * (dtype == DS_F32 ? F32T::kPerLoad : BF16T::kPerLoad);
    prm.tpb = (int32_t)ceil_div(B, te);
    const int64_t items = batch * S;
    if (dtype == DS_F32)
        return vec ? launch<F32T, true, 8>(prm, L.total, hs, items) : launch<F32T, false, 4>(prm, L.total, hs, items);
    return vec ? launch<BF16T, true, 8>(prm, L.total, hs, items) : launch<BF16T, false, 4>(prm, L.total, hs, items);
}

}  // namespace ds

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

int deepselect_validate(int dtype, int64_t batch, int64_t N, int64_t row_stride, int32_t k, int32_t B,
                        int32_t B2) {
    int st = ds::validate_shape(dtype, batch, N, row_stride, k, B, B2);
    if (st != DS_OK) return st;
    if (ds::split_lower_bound(dtype, N, B) > 1 &&
        !ds::split_ok(N, k, B, ds::split_lower_bound(dtype, N, B)))
        return DS_ERR_UNSUPPORTED;
    return ds::lds_check(dtype, N, k, B, B2, ds::split_lower_bound(dtype, N, B));
}

int deepselect_topk(const void* x, int dtype, int64_t batch, int64_t N, int64_t row_stride, int32_t k, int32_t B,
                    int32_t B2, uint64_t seed, void* out_vals, int32_t* out_idx, void* stream) {
    try {
        return ds::topk_impl(x, dtype, batch, N, row_stride, k, B, B2, seed, out_vals, out_idx, stream, nullptr);
    } catch (...) {
        return DS_ERR_HIP;
    }
}

int deepselect_topk_ex(const void* x, int dtype, int64_t batch, int64_t N, int64_t row_stride, int32_t k,
                       int32_t B, int32_t B2, uint64_t seed, void* out_vals, int32_t* out_idx, void* stream,
                       const ds_options_t* opt) {
    try {
        return ds::topk_impl(x, dtype, batch, N, row_stride, k, B, B2, seed, out_vals, out_idx, stream, opt);
    } catch (...) {
        return DS_ERR_HIP;
    }
}

int deepselect_plan_split(int dtype, int64_t batch, int64_t N, int32_t k, int32_t B, int32_t B2,
                          int32_t num_cus) {
    const int st = ds::validate_shape(dtype, batch, N, N, k, B, B2);
    if (st != DS_OK) return st;
    if (num_cus < 1) return DS_ERR_SHAPE;
    return ds::plan_split(dtype, batch, N, k, B, B2, num_cus);
}

size_t deepselect_workspace_bytes(int dtype, int64_t batch, int64_t N, int32_t k, int32_t B, int32_t B2,
                                  int32_t split) {
    if (ds::validate_shape(dtype, batch, N, N, k, B, B2) != DS_OK || split < 1) return 0;
    return ds::make_ws_layout(batch, k, split).total;
}

size_t deepselect_lds_bytes(int dtype, int64_t N, int32_t k, int32_t B, int32_t B2, int32_t split) {
    if (ds::validate_shape(dtype, 1, N, N, k, B, B2) != DS_OK || split < 1) return 0;
    return ds::make_layout(dtype, N, k, B, B2, split).total;
}

const char* deepselect_status_string(int status) {
    switch (status) {
        case DS_OK: return "ok";
        case DS_ERR_NULL: return "a required pointer is NULL";
        case DS_ERR_DTYPE: return "dtype must be DS_F32 or DS_BF16";
        case DS_ERR_SHAPE: return "bad shape: need batch >= 0, 1 <= N < 2^31, row_stride >= N, aligned x";
        case DS_ERR_K: return "k must satisfy 1 <= k <= N";
        case DS_ERR_BLOCK: return "B and B2 must be >= 1 and a forced split must leave every part >= k elements";
        case DS_ERR_UNSUPPORTED: return "candidate buffer k+B+B2 (or the block order) does not fit in LDS";
        case DS_ERR_HIP: return "a HIP call failed";
        case DS_ERR_WORKSPACE: return "caller workspace is smaller than deepselect_workspace_bytes";
        default: return "unknown status";
    }
}

void deepselect_release(void) {
    std::lock_guard<std::mutex> lk(ds::g_mu);
    for (auto& kv : ds::g_ws) {
        if (kv.second.ptr) (void)hipFree(kv.second.ptr);
    }
    ds::g_ws.clear();
}

}  // extern "C"
