// deepselect.hip -- MI355X (gfx950) DeepSelect batched row-wise top-k and its C ABI.
//
// DeepSelect (DeepSelect deep-dive, PFCCLab/DeepSelect, section "算法"): each row
// is read once, in B-element blocks taken in a random order that does not
// depend on the data. Elements above the threshold T go to an on-chip candidate
// buffer; after any block that leaves k + B2 or more entries, a radix select
// keeps the k largest and T becomes the k-th. A final select returns k. Before
// the first compaction every element is admitted (the page says so right after
// the pseudo-code).
//
// Mapping on gfx950
//   * one workgroup per (row, part) owns the candidate buffer (keys + column
//     indices, or packed key/column words for bfloat16 parts of at most 64K
//     elements), the radix histograms and the block order in LDS;
//   * ring kernel (the usual path): each wave owns whole blocks. A step hands
//     the next NW blocks of the order to the NW waves; blocks travel HBM ->
//     LDS with buffer loads that write LDS directly, into a ring of slots per
//     wave, and a step waits only for its own block. Each wave counts its
//     elements above T; one barrier exchanges the NW counts, after which every
//     wave knows where its survivors go and whether some block of the step
//     ends with the buffer at k + B2 or more. If so, the buffer is compacted
//     right after that block and the later blocks of the step are counted
//     again against the new T, so the result and every statistic are those of
//     the block-by-block loop of the pages;
//   * register-streaming kernel: the same step loop with blocks held in
//     registers, Q steps of loads in flight (when the ring does not fit LDS);
//   * generic kernel (unaligned rows, ragged N, blocks over 8 KiB): the whole
//     workgroup shares each block, one barrier per 4 KiB tile;
//   * split rows (the deep-dive's "实现" section, last paragraph: a row cut into
//     parts whose top-k go to one reducer): each part writes its results, their
//     count, its k-th and its largest key to a device workspace; a second
//     kernel, queued behind the first on the same stream, runs DeepSelect over
//     the parts' results (one block per part, parts whose largest key cannot
//     reach the row's top k counted empty without being read) and writes the
//     row. The kernel boundary makes the parts' writes visible. Rows of two
//     bfloat16 parts (unsorted output) are merged instead by the part that
//     ends last, after a device-scope acquire-release count of the row's
//     ended parts: it starts as soon as its own select ends, not after the
//     slowest part of every row, and no second kernel is launched;
//   * the kernel that writes a row can sort its results (a bitonic network in
//     registers and LDS), take a softmax and draw a sample from them; rows may
//     have their own valid lengths; the parts of a split row may share their
//     thresholds (a device-scope atomic maximum per row).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <map>
#include <atomic>
#include <mutex>
#include <thread>
#include <tuple>
#include <utility>

#include "../../include/deepselect.h"
#include "ds_device.hpp"
#include "ds_plan.hpp"
#include "ds_workspace.hpp"

namespace ds {

constexpr uint32_t kOob = 0x80000000u;  // buffer offset past every part (parts < 2 GiB)
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr int kAgentCoherent = 16;  // buffer load cache policy: coherent at device scope
constexpr int64_t kShareMinSteps = 6;  // ring steps per wave below which threshold sharing is off

struct Params {
    const void* x;
    void* out_vals;
    int32_t* out_idx;
    uint64_t* stats;
    uint32_t* ws_keys;
    uint32_t* ws_idx;
    uint64_t* ws_stats;
    int64_t batch, n, row_stride, m;
    uint64_t seed;
    int32_t k, B, B2, split;
    int32_t sorted;  // write each row's results in descending order
    const int32_t* lengths;  // per-row valid lengths (NULL: every row has n)
    float* probs;            // softmax of each row's results (sorted output), or NULL
    const float* sample_u;   // one uniform per row for the sample, or NULL
    int32_t* sample_idx;     // the sampled column of each row
    float inv_temp, top_p;
    uint64_t* ws_share;      // per row: the largest part threshold key + 1 (0: none), or NULL
    uint32_t* ws_cnt;        // per part: its number of results
    uint32_t* ws_tkey;       // per part: its k-th key when it has k results, else 0
    uint32_t* ws_tmax;       // per part: its largest result key (0 without results)
    Layout L;
    uint64_t* ws_arrive;     // per row: parts ended (word kArriveWord of its cell), or NULL: merge kernel
};

// Optional cycle accounting (builds with -DDS_PROFILE only): each wave adds
// the shader-clock cycles between probes to the category of the phase that
// just ended and leaves them in ds_prof[workgroup][wave][category].
#ifdef DS_PROFILE
constexpr int kProfCats = 16, kProfWaves = 8, kProfGroups = 4096;
__device__ unsigned long long ds_prof[kProfGroups * kProfWaves * kProfCats];
#define DS_PROF(st, cat) (st).prof_mark(cat)
#else
#define DS_PROF(st, cat) ((void)0)
#endif

struct RunState {
#ifdef DS_PROFILE
    uint64_t pt_last = __builtin_amdgcn_s_memtime();
    uint64_t pt[kProfCats] = {};
    __device__ void prof_mark(int cat) {
        const uint64_t now = __builtin_amdgcn_s_memtime();
        pt[cat] += now - pt_last;
        pt_last = now;
    }
    __device__ void prof_flush(unsigned group0 = 0) {
        if ((threadIdx.x & 63) == 0 && group0 + blockIdx.x < (unsigned)kProfGroups) {
            unsigned long long* o =
                ds_prof + ((size_t)(group0 + blockIdx.x) * kProfWaves + (threadIdx.x >> 6)) * kProfCats;
            for (int i = 0; i < kProfCats; ++i) atomicAdd(&o[i], (unsigned long long)pt[i]);
        }
    }
#endif
    uint32_t len = 0;   // candidate entries
    bool tset = false;  // threshold set (a compaction happened)
    uint32_t tkey = 0;  // threshold key
    uint64_t W = 0;     // RadixSelectTopK input (can pass 2^32 for huge k / tiny B2)
    uint32_t A = 0, R = 0, maxlen = 0;
    uint32_t par = 0;   // count-buffer parity
    uint32_t kmax = 0;  // the largest key this lane appended (reduced over the wave at a select)
    bool fset = false;  // a threshold filters the blocks (T, or one shared by another part)
    uint32_t fkey = 0;  // its key: the larger of T and the shared one
};

template <class D>
struct Lds {
    typename D::Key* keys;
    uint32_t* idx;
    uint32_t* hist;
    uint32_t* fold;
    uint32_t* tot;
    uint32_t* gathered;
    uint32_t* cnt;
    uint16_t* perm;
    uint32_t* misc;  // [2] gathered-key counter, [8 + w] wave w's largest appended key
                     // (when sorting the results: [8 + w] and [16 + w] wave w's smallest
                     // and largest result key),
                     // [16, 32) four copies of the row's shared threshold cell
                     // (16 bytes each, the cell in the first 8)
    unsigned char* base;
    uint32_t junk;   // first junk entry of the candidate arrays
};

template <class D>
__device__ __forceinline__ Lds<D> lds_of(unsigned char* smem, const Layout& L) {
    Lds<D> s;
    s.base = smem;
    s.keys = reinterpret_cast<typename D::Key*>(smem + L.keys);
    s.idx = reinterpret_cast<uint32_t*>(smem + L.idx);
    s.hist = reinterpret_cast<uint32_t*>(smem + L.hist);
    s.fold = reinterpret_cast<uint32_t*>(smem + L.fold);
    s.tot = reinterpret_cast<uint32_t*>(smem + L.tot);
    s.gathered = reinterpret_cast<uint32_t*>(smem + L.gather);
    s.cnt = reinterpret_cast<uint32_t*>(smem + L.cnt);
    s.perm = reinterpret_cast<uint16_t*>(smem + L.perm);
    s.misc = reinterpret_cast<uint32_t*>(smem + L.misc);
    s.junk = (uint32_t)L.junk;
    return s;
}

// Start of a (row, part): clear the histogram copies (the block order, built
// next, ends with a barrier).
template <class D, int NW>
__device__ __forceinline__ void begin_item(Lds<D>& s) {
    clear_words<NW>(s.hist, kHistWords);
}

// Fold the largest key this lane appended into its running maximum. The top
// of the key range the radix select starts from is the largest over the lanes
// and waves; it is reduced only when a select needs it. A register, not an LDS
// atomic: the compiler makes every LDS atomic wait for the wave's ring loads
// still in flight.
__device__ __forceinline__ void publish_max(RunState& st, uint32_t kmax) {
    st.kmax = kmax > st.kmax ? kmax : st.kmax;
}

// RadixSelectTopK(buffer, k): the buffer keeps its k largest and T becomes the
// k-th key. Once T is set every candidate is >= T, the bottom of the key range.
template <class D, int NW>
__device__ __forceinline__ void select_buffer(Lds<D>& s, RunState& st, uint32_t k) {
    static_assert(NW <= 8, "one largest-key cell per wave in misc[8..16)");
    const uint32_t lo = st.tset ? st.tkey : 0u;
    const uint32_t wmax = wave_max(st.kmax);
    if (lane_id() == 0) s.misc[8 + wave_id()] = wmax;
    lds_barrier();  // appends and the waves' largest keys are visible
    uint32_t hi = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const uint32_t v = s.misc[8 + i];
        hi = v > hi ? v : hi;
    }
    hi = uniform(hi);
    // the barrier above made the appends visible: the select starts without one
#ifdef DS_PROFILE
    st.tkey = select_topk<D, NW>(s.keys, s.idx, s.hist, s.fold, s.tot, s.gathered, s.misc + 2, s.junk, st.len, k, lo,
                                  hi > lo ? hi : lo, true, true, [&](int c) { st.prof_mark(c); });
#else
    st.tkey = select_topk<D, NW>(s.keys, s.idx, s.hist, s.fold, s.tot, s.gathered, s.misc + 2, s.junk, st.len, k, lo,
                                  hi > lo ? hi : lo, true, true);
#endif
    st.tset = true;
    st.fkey = st.fset && st.fkey > st.tkey ? st.fkey : st.tkey;
    st.fset = true;
    st.len = k;
}

// Compaction inside the loop (counts in W and R).
template <class D, int NW>
__device__ __forceinline__ void compact(Lds<D>& s, RunState& st, uint32_t k) {
    DS_PROF(st, 14);
    st.W += st.len;
    st.R += 1;
    select_buffer<D, NW>(s, st, k);
    DS_PROF(st, 13);
}

// Final RadixSelectTopK (its input length counts in W); ends with a barrier.
// With drop_shared, a filter key that another part raised above this part's
// own T first drops the entries at or below it (appended before the key was
// known): the row's k largest are among the other part's results and this
// part's keys above the key, so the select, if one is still needed, runs on
// what is left (W still counts the whole buffer, so W = A + k R holds).
template <class D, int NW>
__device__ __forceinline__ void final_select(Lds<D>& s, RunState& st, uint32_t k, bool drop_shared = false) {
    st.W += st.len;
    if (drop_shared && st.len > 0u && st.fset && (!st.tset || st.fkey > st.tkey)) {
        lds_barrier();  // the appends are visible
        st.len = partition_keep<D, NW>(s.keys, s.idx, s.tot, st.len, st.fkey, 0u, s.junk);
    }
    if (st.len > k) select_buffer<D, NW>(s, st, k);
    lds_barrier();
}

// ===========================================================================
// Streaming kernel: each wave owns whole blocks of U units (one 16-byte load
// per lane per unit; a unit is 64*V elements, V = elements per 16 bytes).
// ===========================================================================
template <int U>
struct BlockRegs {
    u32x4 v[U];
};

// Raw bits of slot q of unit u, and the 32-bit word the threshold test reads
// (bfloat16: the pattern moved to the top half).
template <class D, int U>
__device__ __forceinline__ uint32_t raw_at(const BlockRegs<U>& r, int u, int q) {
    if constexpr (D::kBytes == 4) {
        return r.v[u][q];
    } else {
        const uint32_t d = r.v[u][q >> 1];
        return (q & 1) ? (d >> 16) : (d & 0xFFFFu);
    }
}
template <class D, int U>
__device__ __forceinline__ uint32_t test_word(const BlockRegs<U>& r, int u, int q) {
    if constexpr (D::kBytes == 4) {
        return r.v[u][q];
    } else {
        const uint32_t d = r.v[u][q >> 1];
        return (q & 1) ? d : (d << 16);
    }
}

// A part is streamed in chunks of Q steps; a step hands the next NW blocks of
// the order to the NW waves. All Q loads of a chunk are issued at its start
// into Q register slots, so a wave has Q blocks in flight and pays the memory
// latency about once per chunk. The step loop copies the slot it needs into
// one working block (a uniform branch per slot, so the copy waits only for
// that slot's loads), which keeps one copy of the filter, scatter and
// compaction code and lets the compaction run while later slots still load.
template <class D, int NW, int U, int Q>
struct Streamer {
    static_assert(NW <= 8, "the step's block counts are summed over one 8-lane DPP span");
    static constexpr int V = D::kPerLoad;
    static constexpr int UE = 64 * V;  // elements per unit

    Lds<D>& s;
    RunState& st;
    const __amdgpu_buffer_rsrc_t rsrc;
    const uint32_t part_elem0, part_n, B;  // parts hold < 2^31 bytes
    const int32_t ms, nsteps;
    const uint32_t k, B2;

    // Block at order position bi: element offset inside the part and length.
    __device__ __forceinline__ void block_at(int32_t bi, uint32_t& boff, uint32_t& blen) const {
        if (bi >= ms) {
            boff = 0;
            blen = 0;
            return;
        }
        boff = uniform(s.perm[bi]) * B;
        const uint32_t rem = part_n - boff;
        blen = rem < B ? rem : B;
    }

    __device__ __forceinline__ void load(BlockRegs<U>& r, int32_t bi) const {
        uint32_t boff, blen;
        block_at(bi, boff, blen);
        const uint32_t lane = lane_id();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t e0 = u * UE + lane * V;
            const uint32_t off = e0 < blen ? (boff + e0) * D::kBytes : kOob;
            r.v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
        }
    }

    // Elements past the end of a short block (whole 16-byte loads, or the
    // tail of the load that holds the end) get all-ones bits, whose key is 0:
    // never above any threshold.
    __device__ __forceinline__ void mask_tail(BlockRegs<U>& r, uint32_t blen) const {
        const uint32_t lane = lane_id();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t e0 = u * UE + lane * V;
            const uint32_t nv = e0 < blen ? blen - e0 : 0u;  // the lane's elements inside the block
            if (nv < (uint32_t)V) {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    if constexpr (V == 4)
                        r.v[u][w] |= (uint32_t)w >= nv ? ~0u : 0u;
                    else
                        r.v[u][w] |= ((uint32_t)(2 * w) >= nv ? 0xFFFFu : 0u) |
                                     ((uint32_t)(2 * w + 1) >= nv ? 0xFFFF0000u : 0u);
                }
            }
        }
    }

    // Elements of the block above T (uniform over the wave).
    template <bool kNeg>
    __device__ __forceinline__ uint32_t count_above(const BlockRegs<U>& r, uint32_t thr) const {
        uint32_t c = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int q = 0; q < V; ++q) c += (uint32_t)__popcll(__ballot(above_k<kNeg>(test_word<D, U>(r, u, q), thr)));
        }
        return c;
    }

    // Append every element of the block at base (before the first
    // compaction), in element order.
    __device__ __forceinline__ void scatter_all(const BlockRegs<U>& r, uint32_t base, uint32_t boff,
                                                uint32_t blen) const {
        const uint32_t lane = lane_id();
        const uint32_t col0 = part_elem0 + boff;
        uint32_t kmax = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int q = 0; q < V; ++q) {
                const uint32_t e = u * UE + lane * V + q;
                if (e < blen) {
                    const uint32_t key = D::key(raw_at<D, U>(r, u, q));
                    s.keys[base + e] = (typename D::Key)key;
                    s.idx[base + e] = col0 + e;
                    kmax = key > kmax ? key : kmax;
                }
            }
        }
        publish_max(st, kmax);
    }

    // Append the elements of the block above T at base, in (unit, slot,
    // lane) order.
    template <bool kNeg>
    __device__ __forceinline__ void scatter_above(const BlockRegs<U>& r, uint32_t base, uint32_t boff,
                                                  uint32_t thr) const {
        const uint32_t col0 = part_elem0 + boff + lane_id() * V;
        uint32_t kmax = 0, off = base;
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int q = 0; q < V; ++q) {
                const bool pred = above_k<kNeg>(test_word<D, U>(r, u, q), thr);
                const uint64_t m = __ballot(pred);
                if (m != 0ull) {
                    if (pred) {
                        const uint32_t pos = off + lanes_below(m);
                        const uint32_t key = D::key(raw_at<D, U>(r, u, q));
                        s.keys[pos] = (typename D::Key)key;
                        s.idx[pos] = col0 + (uint32_t)(u * UE + q);
                        kmax = key > kmax ? key : kmax;
                    }
                    off += (uint32_t)__popcll(m);
                }
            }
        }
        publish_max(st, kmax);
    }

    // Copy slot j into the working block: a chain of uniform branches, one per
    // slot, so the copy of slot q waits only for the loads of slot q. The asm
    // statement that ends each branch names its slot as an immediate, which
    // keeps the compiler from merging the branches into one copy from a
    // variable slot index (that would put the slots in scratch memory).
    template <int q>
    __device__ __forceinline__ void take(BlockRegs<U> (&slots)[Q], int32_t j, BlockRegs<U>& r) const {
        if constexpr (q < Q) {
            if (j == q) {
                r = slots[q];
#pragma unroll
                for (int u = 0; u < U; ++u) asm volatile("; slot %1" : "+v"(r.v[u]) : "i"(q));
            } else {
                take<q + 1>(slots, j, r);
            }
        }
    }

    // Blocks first..nblk-1 of the step, counted against the current state:
    // publish the counts, then append them in order up to (and including) the
    // first block after which the buffer holds k + B2 or more. Returns that
    // block's wave, or -1 when every block was appended without reaching it.
    __device__ __forceinline__ int32_t append_from(const BlockRegs<U>& r, uint32_t boff, uint32_t blen,
                                                   int32_t first, int32_t nblk) {
        const int w = wave_id();
        const bool mine = w >= first && w < nblk;
        uint32_t c = 0;
        Thresh th{};
        if (mine) {
            if (!st.fset) {
                c = blen;
            } else {
                th = make_thresh<D>(st.fkey);
                c = th.neg ? count_above<true>(r, th.thr) : count_above<false>(r, th.thr);
            }
        }
        if (lane_id() == 0) s.cnt[st.par * NW + w] = c;
        lds_barrier();
        // the pages' order: block after block, compaction check after each.
        // Lane g < NW takes block g's count (0 outside [first, nblk)); a
        // prefix sum over those lanes gives the length after each block, the
        // first lane reaching k + B2 is the trigger.
        const int32_t lid = (int32_t)lane_id();
        const bool inb = lid >= first && lid < nblk;
        const uint32_t cg = inb ? s.cnt[st.par * NW + lid] : 0u;
        st.par ^= 1u;
        uint32_t inc = cg;  // inclusive prefix over lanes 0..NW-1 (one DPP row)
        inc += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)inc, 0x111, 0xF, 0xF, true);  // row_shr:1
        inc += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)inc, 0x112, 0xF, 0xF, true);  // row_shr:2
        inc += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)inc, 0x114, 0xF, 0xF, true);  // row_shr:4
        const uint64_t over = __ballot(inb && st.len + inc >= k + B2);
        const int32_t trig = over != 0ull ? (int32_t)__builtin_ctzll(over) : -1;
        const int32_t last = trig >= 0 ? trig : nblk - 1;
        const uint32_t run = st.len + uniform(__builtin_amdgcn_readlane(inc, last));
        const uint32_t my_base = st.len + uniform(__builtin_amdgcn_readlane(inc - cg, w));
        if (mine && w <= last && c != 0) {
            if (!st.fset)
                scatter_all(r, my_base, boff, blen);
            else if (th.neg)
                scatter_above<true>(r, my_base, boff, th.thr);
            else
                scatter_above<false>(r, my_base, boff, th.thr);
        }
        st.A += run - st.len;
        st.maxlen = run > st.maxlen ? run : st.maxlen;
        st.len = run;
        return trig;
    }

    __device__ __forceinline__ void run() {
        const int w = wave_id();
        for (int32_t c0 = 0; c0 < nsteps; c0 += Q) {
            BlockRegs<U> slots[Q];
#pragma unroll
            for (int q = 0; q < Q; ++q) load(slots[q], (c0 + q) * NW + w);
            const int32_t nst = nsteps - c0 < Q ? nsteps - c0 : Q;
            int32_t j = 0, first = 0;
            BlockRegs<U> r;
            uint32_t boff = 0, blen = 0;
            while (j < nst) {
                const int32_t stp = c0 + j;
                const int32_t nblk = ms - stp * NW < NW ? ms - stp * NW : NW;  // blocks in this step
                if (first == 0) {
                    block_at(stp * NW + w, boff, blen);
                    if (w < nblk) {
                        take<0>(slots, j, r);
                        if (blen != U * UE) mask_tail(r, blen);
                    }
                }
                const int32_t trig = append_from(r, boff, blen, first, nblk);
                if (trig >= 0) {
                    compact<D, NW>(s, st, k);
                    if (trig < nblk - 1) {
                        first = trig + 1;  // the blocks behind it, against the new T
                        continue;
                    }
                }
                ++j;
                first = 0;
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Ring streaming: blocks travel HBM -> LDS with buffer loads that write LDS
// directly (no registers held while they fly), into a ring of `depth` block
// slots per wave. A step waits (vmcnt) only for its own block, reads it into
// registers, and refills the slot with the block `depth` steps ahead.
// ---------------------------------------------------------------------------
// s_waitcnt that waits until at most N vector-memory operations are
// outstanding and leaves the other counters alone.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt for every outstanding LDS operation of the wave.
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

template <class D, int NW, int U>
struct RingStreamer {
    static_assert(NW <= 8, "the step's block counts are summed over one 8-lane DPP span");
    static constexpr int V = D::kPerLoad;
    static constexpr int UE = 64 * V;  // elements per unit
    static constexpr bool kPk = is_packed<D>::value;
    static_assert(!kPk || V == 8, "packed entries are bfloat16 candidates");

    // Store candidate (key, column col inside the part) at buffer position at:
    // one packed entry, or the key and the row column in their two arrays.
    __device__ __forceinline__ void put(uint32_t at, uint32_t key, uint32_t col) const {
        if constexpr (kPk) {
            s.keys[at] = (key << 16) | col;
        } else {
            s.keys[at] = (typename D::Key)key;
            s.idx[at] = part_elem0 + col;
        }
    }

    Lds<D>& s;
    RunState& st;
    const __amdgpu_buffer_rsrc_t rsrc;
    const uint32_t part_elem0, part_n, B;  // parts hold < 2^31 bytes
    const int32_t ms, nsteps, depth;
    const uint32_t k, B2;
    u32x4* ring;  // this wave's slots: slot q unit u at ring[(q*U + u)*64 + lane]
    uint64_t* share;  // the row's shared threshold cell (key + 1, 0: none), or NULL

    __device__ __forceinline__ void block_at(int32_t bi, uint32_t& boff, uint32_t& blen) const {
        if (bi >= ms) {
            boff = 0;
            blen = 0;
            return;
        }
        boff = uniform(s.perm[bi]) * B;
        const uint32_t rem = part_n - boff;
        blen = rem < B ? rem : B;
    }

    // Start copying the block at order position bi into slot q (U buffer
    // loads of 16 bytes per lane; lanes past the block read nothing).
    __device__ __forceinline__ void fetch(int32_t bi, int32_t q) const {
        uint32_t boff, blen;
        block_at(bi, boff, blen);
        const uint32_t lane = lane_id();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t e0 = u * UE + lane * V;
            const uint32_t off = e0 < blen ? (boff + e0) * D::kBytes : kOob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (__attribute__((address_space(3))) void*)(ring + (q * U + u) * 64), 16, off, 0, 0, 0);
        }
    }

    // Wait until the block with `ahead` blocks fetched after it has landed.
    __device__ __forceinline__ void wait_block(int32_t ahead) const {
        if (ahead <= 0)
            wait_vm<0>();
        else if (ahead == 1)
            wait_vm<U>();
        else if (ahead == 2)
            wait_vm<2 * U>();
        else
            wait_vm<3 * U>();
    }

    __device__ __forceinline__ void read_slot(int32_t q, BlockRegs<U>& r) const {
        const uint32_t lane = lane_id();
#pragma unroll
        for (int u = 0; u < U; ++u) r.v[u] = ring[(q * U + u) * 64 + lane];
    }

    // Elements past the end of a short block (whole 16-byte loads, or the
    // tail of the load that holds the end) get all-ones bits, whose key is 0:
    // never above any threshold.
    __device__ __forceinline__ void mask_tail(BlockRegs<U>& r, uint32_t blen) const {
        const uint32_t lane = lane_id();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t e0 = u * UE + lane * V;
            const uint32_t nv = e0 < blen ? blen - e0 : 0u;  // the lane's elements inside the block
            if (nv < (uint32_t)V) {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    if constexpr (V == 4)
                        r.v[u][w] |= (uint32_t)w >= nv ? ~0u : 0u;
                    else
                        r.v[u][w] |= ((uint32_t)(2 * w) >= nv ? 0xFFFFu : 0u) |
                                     ((uint32_t)(2 * w + 1) >= nv ? 0xFFFF0000u : 0u);
                }
            }
        }
    }

    // This lane's elements above T as a bit mask (element u*V + q of the lane
    // at bit u*V + q; blocks of more than 32 elements per lane keep only the
    // count, in the low bits, with bit 31 set), one 32-bit compare per element
    // (the threshold's sign fixed at compile time).
    static constexpr bool kMasks = U * V <= 32;
    // bfloat16 masks hold the low halves of the lane's words in bits 0-15 and
    // the high halves in bits 16-31 (element q of unit u: word u*4 + q/2,
    // half q%2), so one packed 16-bit test gives a word's two bits at once;
    // float32 masks (and 64-bit ones) hold element q of unit u at u*V + q.
    static constexpr bool kPkMask = D::kBytes == 2 && kMasks;
    static __device__ __forceinline__ constexpr int mask_bit(int u, int q) {
        return kPkMask ? ((q & 1) * 16 + u * 4 + (q >> 1)) : (u * V + q);
    }
    template <bool kNeg>
    __device__ __forceinline__ uint32_t lane_mask(const BlockRegs<U>& r, uint32_t thr) const {
        if constexpr (kPkMask) {
            // Both halves of a word against the threshold's 16 bits with one
            // saturating packed subtract whose sign bits are the tests: above
            // a threshold at or over +0, t - h < 0 (signed halves); below a
            // negative one's bits, (h ^ 0x8000) - (t ^ 0x8000) < 0 (unsigned
            // order as signed). The same tests as above_k on the two words.
            typedef short s2 __attribute__((ext_vector_type(2)));
            const uint32_t t16 = thr >> 16;
            const s2 tv = kNeg ? s2{(short)(t16 ^ 0x8000u), (short)(t16 ^ 0x8000u)} : s2{(short)t16, (short)t16};
            uint32_t m = 0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int wi = u * 4 + w;
                    const uint32_t d = r.v[u][w];
                    const s2 sv = kNeg ? __builtin_elementwise_sub_sat(__builtin_bit_cast(s2, d ^ 0x80008000u), tv)
                                       : __builtin_elementwise_sub_sat(tv, __builtin_bit_cast(s2, d));
                    const uint32_t sb = __builtin_bit_cast(uint32_t, sv);
                    m |= (sb >> (15 - wi)) & ((1u << wi) | (1u << (16 + wi)));
                }
            }
            return m;
        }
        uint32_t m = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int q = 0; q < V; ++q) {
                const bool p = above_k<kNeg>(test_word<D, U>(r, u, q), thr);
                if constexpr (kMasks)
                    m |= p ? 1u << (u * V + q) : 0u;
                else
                    m += p ? 1u : 0u;
            }
        }
        return m;
    }
    __device__ __forceinline__ static uint32_t mask_count(uint32_t m) {
        if constexpr (kMasks)
            return (uint32_t)__builtin_popcount(m);
        else
            return m;
    }

    // This lane's elements inside the block (every element is admitted before
    // the first compaction).
    __device__ __forceinline__ uint32_t lane_valid(uint32_t blen) const {
        const uint32_t lane = lane_id();
        uint32_t c = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t e0 = u * UE + lane * V;
            c += e0 >= blen ? 0u : (blen - e0 < (uint32_t)V ? blen - e0 : (uint32_t)V);
        }
        return c;
    }

    // Append this lane's admitted elements at pos, in element order (lanes in
    // order, so the wave's survivors fill [base, base + count) lane by lane).
    // A slot that admits nothing in the whole wave is skipped; otherwise the
    // lanes that do not admit it store to their junk entry.
    // Key of every element of a 32-bit word (bfloat16: both halves).
    __device__ __forceinline__ static uint32_t word_keys(uint32_t d) {
        if constexpr (D::kBytes == 4) {
            return key_f32(d);
        } else {
            const uint32_t neg = ((d >> 15) & 0x00010001u) * 0xFFFFu;
            return d ^ (neg | 0x80008000u);
        }
    }
    __device__ __forceinline__ static uint32_t word_max(uint32_t kw) {
        if constexpr (D::kBytes == 4) {
            return kw;
        } else {
            const uint32_t lo = kw & 0xFFFFu, hi = kw >> 16;
            return lo > hi ? lo : hi;
        }
    }

    // Append every element inside the block (before the first compaction).
    __device__ __forceinline__ void scatter_valid(const BlockRegs<U>& r, uint32_t pos, uint32_t boff,
                                                  uint32_t blen) const {
        uint32_t lane = lane_id();
        asm volatile("" : "+v"(lane));  // nothing here may be hoisted out of the retry loop
        const uint32_t col0 = boff + lane * V;
        const uint32_t junk = s.junk + lane;
        uint32_t kmax = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int q = 0; q < V; ++q) {
                const bool pred = u * UE + lane * V + q < blen;
                const uint32_t key = D::key(raw_at<D, U>(r, u, q));
                const uint32_t at = pred ? pos : junk;
                put(at, key, col0 + (uint32_t)(u * UE + q));
                pos += pred ? 1u : 0u;
                kmax = pred && key > kmax ? key : kmax;
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        publish_max(st, kmax);
    }

    // Append the lane's elements above T (mask m) at pos in element order:
    // element b of the lane goes to pos plus the number of admitted elements
    // before it (a bit count of the mask), so the stores do not wait on each
    // other; lanes that do not admit it store to their junk entry. With T at
    // or above +0 (kPos) every admitted element is positive and its key is
    // its bits with the sign bit set. The largest key appended is the block's
    // largest key, since that one is admitted whenever any is.
    template <bool kPos, class MaskT>
    __device__ __forceinline__ void scatter_dense(const BlockRegs<U>& r, MaskT m, uint32_t pos,
                                                  uint32_t boff) const {
        uint32_t lane = lane_id();
        asm volatile("" : "+v"(lane));
        const uint32_t col0 = boff + lane * V;
        const uint32_t junk = s.junk + lane;
        constexpr uint32_t kSign = D::kBytes == 4 ? 0x80000000u : 0x80008000u;
        uint32_t kmax = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t kw = kPos ? (r.v[u][w] ^ kSign) : word_keys(r.v[u][w]);
                const uint32_t wm = word_max(kw);
                kmax = wm > kmax ? wm : kmax;
#pragma unroll
                for (int h = 0; h < V / 4; ++h) {
                    const int q = w * (V / 4) + h;
                    const int b = sizeof(MaskT) == 4 ? mask_bit(u, q) : u * V + q;
                    const bool pred = (m >> b) & 1;
                    uint32_t before;
                    if constexpr (sizeof(MaskT) == 8)
                        before = (uint32_t)__builtin_popcountll(m & ((1ull << b) - 1ull));
                    else
                        before = (uint32_t)__builtin_popcount((uint32_t)m & ((1u << b) - 1u));
                    const uint32_t at = pred ? pos + before : junk;
                    const uint32_t col = col0 + (uint32_t)(u * UE + q);
                    if constexpr (kPk) {
                        s.keys[at] = (h ? (kw & 0xFFFF0000u) : (kw << 16)) | col;
                    } else {
                        s.keys[at] = (typename D::Key)(h ? kw >> 16 : kw);
                        s.idx[at] = part_elem0 + col;
                    }
                }
            }
        }
        publish_max(st, kmax);
    }

    // Few survivors in the wave (c <= 64): every lane walks its own admitted
    // elements (mask m) lowest first and appends each at pos, reading its raw
    // bits back from the block's ring slot (the loop runs as often as the
    // lane with the most survivors needs).
    __device__ __forceinline__ void scatter_few(uint32_t m, uint32_t pos, uint32_t boff, const u32x4* slot) const {
        uint32_t lane = lane_id();
        asm volatile("" : "+v"(lane));
        const unsigned char* lp = reinterpret_cast<const unsigned char*>(slot + lane);
        const uint32_t col0 = boff + lane * V;
        uint32_t kmax = 0;
        while (m != 0u) {
            const uint32_t e = (uint32_t)__builtin_ctz(m);
            m &= m - 1u;
            uint32_t u, q;  // the element of bit e (mask_bit's inverse)
            if constexpr (kPkMask) {
                u = (e & 15u) >> 2;
                q = ((e & 3u) << 1) | (e >> 4);
            } else {
                u = e / V;
                q = e % V;
            }
            const unsigned char* p = lp + u * (64 * 16) + q * D::kBytes;
            const uint32_t raw = D::kBytes == 4 ? *reinterpret_cast<const uint32_t*>(p)
                                                : (uint32_t)*reinterpret_cast<const uint16_t*>(p);
            const uint32_t key = D::key(raw);
            put(pos, key, col0 + u * UE + q);
            ++pos;
            kmax = key > kmax ? key : kmax;
        }
        publish_max(st, kmax);
    }

    // Append a whole full block at pos (before the first compaction, when
    // pos is a multiple of 8): lane l's U*V elements go to pos + l*U*V in its
    // element order with 16-byte stores, keys transformed a 32-bit word at a
    // time.
    __device__ __forceinline__ void append_full(const BlockRegs<U>& r, uint32_t pos, uint32_t boff) const {
        uint32_t lane = lane_id();
        asm volatile("" : "+v"(lane));  // nothing here may be hoisted out of the retry loop
        const uint32_t at0 = pos + lane * (U * V);
        const uint32_t col0 = (kPk ? 0u : part_elem0) + boff + lane * V;
        uint32_t kmax = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t at = at0 + u * V;
            u32x4 kw;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t d = r.v[u][q];
                uint32_t key;
                if constexpr (D::kBytes == 4) {
                    key = key_f32(d);
                    kmax = key > kmax ? key : kmax;
                } else {
                    // both halves: flip every bit of a negative pattern, the sign bit otherwise
                    const uint32_t neg = ((d >> 15) & 0x00010001u) * 0xFFFFu;
                    key = d ^ (neg | 0x80008000u);
                    const uint32_t lo = key & 0xFFFFu, hi = key >> 16;
                    const uint32_t m = lo > hi ? lo : hi;
                    kmax = m > kmax ? m : kmax;
                }
                kw[q] = key;
            }
            const uint32_t c = col0 + u * UE;
            if constexpr (kPk) {
                // entries key << 16 | column, two 16-byte stores per 8 elements
                *reinterpret_cast<u32x4*>(&s.keys[at]) =
                    u32x4{(kw[0] << 16) | c, (kw[0] & 0xFFFF0000u) | (c + 1), (kw[1] << 16) | (c + 2),
                          (kw[1] & 0xFFFF0000u) | (c + 3)};
                *reinterpret_cast<u32x4*>(&s.keys[at + 4]) =
                    u32x4{(kw[2] << 16) | (c + 4), (kw[2] & 0xFFFF0000u) | (c + 5), (kw[3] << 16) | (c + 6),
                          (kw[3] & 0xFFFF0000u) | (c + 7)};
            } else {
                *reinterpret_cast<u32x4*>(&s.keys[at]) = kw;
#pragma unroll
                for (int h = 0; h < V / 4; ++h)
                    *reinterpret_cast<u32x4*>(&s.idx[at + 4 * h]) =
                        u32x4{c + 4 * h, c + 4 * h + 1, c + 4 * h + 2, c + 4 * h + 3};
            }
        }
        publish_max(st, kmax);
    }

    // Blocks first..nblk-1 of the step counted against the current state, then
    // appended in order up to (and including) the first block after which the
    // buffer holds k + B2 or more. Returns that block's wave, or -1.
    __device__ __forceinline__ int32_t append_from(const BlockRegs<U>& r0, uint32_t boff, uint32_t blen,
                                                   int32_t first, int32_t nblk, const u32x4* slot) {
        // The block passes through an empty asm statement here, so nothing
        // derived from it (keys, shifted words, columns of every slot) can be
        // hoisted out of the step's retry loop and held in registers.
        BlockRegs<U> r = r0;
#pragma unroll
        for (int u = 0; u < U; ++u) asm volatile("" : "+v"(r.v[u]));
        const int w = wave_id();
        const bool mine = w >= first && w < nblk;
        uint32_t lc = 0, lm = 0;
        Thresh th{};
        if (mine) {
            if (!st.fset) {
                lc = lane_valid(blen);
            } else {
                th = make_thresh<D>(st.fkey);
                lm = th.neg ? lane_mask<true>(r, th.thr) : lane_mask<false>(r, th.thr);
                lc = mask_count(lm);
            }
        }
        const uint32_t incl = wave_prefix_sum(lc);
        const uint32_t c = uniform(__builtin_amdgcn_readlane(incl, 63));
        if (lane_id() == 0) s.cnt[st.par * NW + w] = c;
        DS_PROF(st, 2);
        lds_barrier();
        DS_PROF(st, 3);
        // the pages' order: block after block, compaction check after each.
        // Lane g < NW takes block g's count (0 outside [first, nblk)); a
        // prefix sum over those lanes gives the length after each block, the
        // first lane reaching k + B2 is the trigger.
        const int32_t lid = (int32_t)lane_id();
        const bool inb = lid >= first && lid < nblk;
        const uint32_t cg = inb ? s.cnt[st.par * NW + lid] : 0u;
        st.par ^= 1u;
        uint32_t inc = cg;  // inclusive prefix over lanes 0..NW-1 (one DPP row)
        inc += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)inc, 0x111, 0xF, 0xF, true);  // row_shr:1
        inc += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)inc, 0x112, 0xF, 0xF, true);  // row_shr:2
        inc += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)inc, 0x114, 0xF, 0xF, true);  // row_shr:4
        const uint64_t over = __ballot(inb && st.len + inc >= k + B2);
        const int32_t trig = over != 0ull ? (int32_t)__builtin_ctzll(over) : -1;
        const int32_t last = trig >= 0 ? trig : nblk - 1;
        const uint32_t run = st.len + uniform(__builtin_amdgcn_readlane(inc, last));
        const uint32_t my_base = st.len + uniform(__builtin_amdgcn_readlane(inc - cg, w));
        if (mine && w <= last && c != 0) {
            const uint32_t pos = my_base + incl - lc;
            if (!st.fset) {
                if (blen == (uint32_t)(U * UE) && (my_base & 7u) == 0u)
                    append_full(r, my_base, boff);
                else
                    scatter_valid(r, pos, boff, blen);
            } else if (kMasks && c <= 64u) {
                scatter_few(lm, pos, boff, slot);
            } else if (kMasks) {
                if (th.neg)
                    scatter_dense<false>(r, lm, pos, boff);
                else
                    scatter_dense<true>(r, lm, pos, boff);
            } else if (th.neg) {
                scatter_dense<false>(r, lane_bits<true>(r, th.thr), pos, boff);
            } else {
                scatter_dense<true>(r, lane_bits<false>(r, th.thr), pos, boff);
            }
        }
        st.A += run - st.len;
        st.maxlen = run > st.maxlen ? run : st.maxlen;
        st.len = run;
        DS_PROF(st, 4);
        return trig;
    }

    // Per-element admission as a 64-bit mask when a lane holds more than 32
    // elements (the dense scatter then tests bits of it).
    template <bool kNeg>
    __device__ __forceinline__ uint64_t lane_bits(const BlockRegs<U>& r, uint32_t thr) const {
        uint64_t m = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int q = 0; q < V; ++q) m |= above_k<kNeg>(test_word<D, U>(r, u, q), thr) ? 1ull << (u * V + q) : 0ull;
        }
        return m;
    }

    __device__ __forceinline__ void run() {
        const int w = wave_id();
        // Only the first block is requested before the loop: with every
        // workgroup starting at once, the first blocks then come back without
        // queueing behind everyone's later ones. The rest of the ring is
        // requested as soon as the first block has landed.
        int32_t issued = 0;  // steps whose block of this wave is fetched
        if (nsteps > 0) fetch(w, 0), issued = 1;
        BlockRegs<U> r;
        // The row's shared threshold cell: at the start of step s wave 0
        // copies it into LDS copy s % 4 by the same kind of asynchronous load
        // as the blocks (no register waits for it: a use of a value loaded
        // into a register one step earlier gets a wait for every load in
        // flight, the newest block's included). Wave 0's wait for its next
        // block covers the copy, and that step's count exchange barrier
        // comes after the wait, so every wave reads copy s % 4 after the
        // appends of step s + 1 and filters with it from step s + 2: one read
        // of the cell per workgroup and step, and the same filter key in
        // every wave. Wave 0 rewrites the copy at step s + 4, after the
        // barrier of step s + 2 that every wave reaches with its read done.
        const __amdgpu_buffer_rsrc_t cell =
            __builtin_amdgcn_make_buffer_rsrc(share, (short)0, 8, (int)kRsrcWord3);
        const uint32_t* copies = s.misc + 16;
        uint32_t sh_lo = 0, sh_hi = 0;  // the cell as copied two steps before this one
        uint64_t told = 0;              // the last T this part published, + 1 (thread 0)
        for (int32_t stp = 0; stp < nsteps; ++stp) {
            const int32_t q = stp % depth;
            const int32_t nblk = ms - stp * NW < NW ? ms - stp * NW : NW;  // blocks in this step
            uint32_t boff, blen;
            block_at(stp * NW + w, boff, blen);
            DS_PROF(st, 14);
            wait_block(issued - 1 - stp);
            read_slot(q, r);
            DS_PROF(st, 1);
            if (share) {
                const uint64_t shared = uniform(sh_lo) | ((uint64_t)uniform(sh_hi) << 32);
                if (shared != 0u) {
                    // another part's threshold (any part's k-th is at most
                    // the row's) raises the filter of this wave's blocks
                    const uint32_t key = (uint32_t)(shared - 1u);
                    if (!st.fset || key > st.fkey) st.fkey = key, st.fset = true;
                }
                // The part's T goes out when it is above what the cell held,
                // and wave 0 copies the cell: both issued here, a step's work
                // before wave 0's next wait for a block.
                const uint64_t mine = st.tset ? (uint64_t)st.tkey + 1u : 0u;
                if (threadIdx.x == 0 && mine > told && mine > shared) {
                    __hip_atomic_fetch_max(share, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    told = mine;
                }
                if (stp + 2 < nsteps && threadIdx.x < 2u)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        cell, (__attribute__((address_space(3))) void*)(copies + 4 * (stp & 3)), 4, threadIdx.x * 4u,
                        0, 0, kAgentCoherent);
            }
            if (stp == 0) {
                for (; issued < depth && issued < nsteps; ++issued) fetch(issued * NW + w, issued);
            }
            if (w < nblk && blen != U * UE) mask_tail(r, blen);
            int32_t first = 0;
            while (true) {
                const int32_t trig = append_from(r, boff, blen, first, nblk, ring + q * U * 64);
                if (trig < 0) break;
                compact<D, NW>(s, st, k);
                if (trig >= nblk - 1) break;
                first = trig + 1;  // the blocks behind it, against the new T
            }
            if (share && stp >= 1 && stp + 1 < nsteps) {
                // the copy wave 0 made at the previous step's start, for the next step
                const u32x4 c = *reinterpret_cast<const u32x4*>(copies + 4 * ((stp - 1) & 3));
                sh_lo = c[0];
                sh_hi = c[1];
            }
            if (issued < nsteps) {
                wait_lgkm();  // this wave's reads of slot q are done before it is refilled
                fetch(issued * NW + w, q);
                ++issued;
            }
        }
    }
};

template <class D, int NW, int U>
__global__ __launch_bounds__(NW * 64) void deepselect_ring_kernel(Params p);

// The kernel's arguments read again from the kernel argument segment (Params
// is a kernel's only explicit argument, at the segment's start), behind an
// empty asm the compiler cannot look through, so that these loads are not
// hoisted to the kernel's start: values used only at a part's end then do
// not stay live through the step loop, where they would be spilled (the ring
// kernels' scalar spills fall from about 180 to 80-130).
__device__ __forceinline__ Params reload_params() {
#if defined(__HIP_DEVICE_COMPILE__)
    auto kp = (const __attribute__((address_space(4))) Params*)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(kp));
    return *kp;
#else
    return Params{};
#endif
}

// Rows of two parts merged inside the part kernel, by the part that ends
// last. Each part has written its results, counts and statistics; after a
// workgroup barrier (every thread's stores done) thread 0 counts the part in
// the row's arrival word with a device-scope acquire-release add, which
// publishes this workgroup's stores and, for the part that sees the other
// part already counted, makes that part's stores visible to its loads. The
// last part resets the word for the next call. Returns whether this part
// merges the row (the same in every thread).
__device__ __forceinline__ bool arrive_last(const Params& p, int64_t row, uint32_t* flag) {
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t* w = p.ws_arrive + row * kCellWords;
        const uint64_t before = __hip_atomic_fetch_add(w, 1ull, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = before + 1u == (uint64_t)p.split;
        if (last) __hip_atomic_store(w, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = last ? 1u : 0u;
    }
    lds_barrier();
    return uniform(*flag) != 0u;
}
template <int NW>
__device__ void merge_in_part_kernel(unsigned char* smem, const Params& p, int64_t row);

// Sorted output. Every result becomes one 64-bit word key << 32 | ~column,
// so plain descending order of the words is the wanted one (keys from the
// largest down, equal keys by ascending column); padding words are 0, below
// every result (~column >= 2^31). The words are ordered by Batcher's bitonic
// network, which "CUDA 算子笔记 4" ("Top K Selection", the bitonic approach)
// also sorts its candidates with. In the stage of distance j inside runs of
// `size` words, words i and i ^ j meet; runs whose index has bit `size` clear
// are ordered descending, the others ascending, and the lower index of a pair
// ends with the larger word in a descending run.
__device__ __forceinline__ bool keeps_larger(uint32_t i, uint32_t j, uint32_t size) {
    return ((i & j) == 0) == ((i & size) == 0);
}

// Plain form: n2 (a power of two) words in LDS at a. Pair q (thread q mod
// NT) joins word i = q with a zero bit inserted at log2(j) and word i + j.
// While j < 64 the 64 pairs a wave takes at once stay inside the same 128
// words whatever j is, so consecutive such stages need only the wave's own
// (in-order) LDS accesses; every other stage waits for the workgroup. Starts
// and ends with a workgroup barrier.
template <int NW>
__device__ __forceinline__ void bitonic_lds(uint64_t* a, uint32_t n2) {
    constexpr uint32_t NT = NW * 64;
    const uint32_t half = n2 >> 1;
    bool local = false;  // the previous stage kept to each wave's words
    for (uint32_t size = 2; size <= n2; size <<= 1) {
        for (uint32_t j = size >> 1; j > 0; j >>= 1) {
            const bool here = j < 64;
            if (here && local)
                asm volatile("" ::: "memory");  // keep the compiler from reordering across stages
            else
                lds_barrier();
            local = here;
            for (uint32_t q = threadIdx.x; q < half; q += NT) {
                const uint32_t i = ((q & ~(j - 1)) << 1) | (q & (j - 1));
                const uint64_t x = a[i], y = a[i + j];
                if ((i & size) == 0 ? x < y : x > y) {
                    a[i] = y;
                    a[i + j] = x;
                }
            }
        }
    }
    lds_barrier();
}

// A stage of distance J < E inside each thread's E words (i0 = E * thread,
// so word i0 + e has bit `size` set when i0 or e has).
// The word of x and o that a side keeping the larger (big) or the smaller
// one ends with: a 32-bit word as the median of x, o and t (t all ones to
// keep the larger, zero to keep the smaller; written as
// max(min(x, o), min(max(x, o), t)), one v_med3_u32, with t shared by the
// words of a stage), a 64-bit one through one compare.
__device__ __forceinline__ uint32_t keep_side(uint32_t x, uint32_t o, bool big) {
    const uint32_t t = big ? 0xFFFFFFFFu : 0u;
    const uint32_t mn = o > x ? x : o, mx = o > x ? o : x;
    const uint32_t c = mx < t ? mx : t;
    return mn > c ? mn : c;
}
__device__ __forceinline__ uint64_t keep_side(uint64_t x, uint64_t o, bool big) {
    return (o > x) == big ? o : x;
}

template <int E, int J, class W>
__device__ __forceinline__ void bitonic_in_thread(W (&v)[E], uint32_t i0, uint32_t size) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if ((e & J) == 0) {
            const W x = v[e], y = v[e | J];
            const bool desc = ((i0 | (uint32_t)e) & size) == 0;
            v[e] = keep_side(x, y, desc);
            v[e | J] = keep_side(y, x, !desc);
        }
    }
}

// The 32-bit word of lane (lane ^ D) of the wave, with vector ALU lane moves
// only: DPP quad permutes (D = 1, 2), a DPP row shift either way (D = 4), a
// DPP row rotation by 8 (D = 8, xor 8 inside a 16-lane row), and the gfx950
// 16- and 32-lane half swaps (D = 16, 32).
template <int D>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
    if constexpr (D == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    } else if constexpr (D == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    } else if constexpr (D == 4) {
        const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x104, 0xF, 0xF, false);  // row_shl:4, lane + 4
        const uint32_t dn = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x114, 0xF, 0xF, false);  // row_shr:4, lane - 4
        return (lane_id() & 4) ? dn : up;
    } else if constexpr (D == 8) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);  // row_ror:8
    } else if constexpr (D == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane_id() & 16) ? r[0] : r[1];
    } else {
        static_assert(D == 32, "lane distance");
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane_id() & 32) ? r[0] : r[1];
    }
}

// A stage of distance j = D * E: word e of this lane meets word e of lane
// (lane ^ D); all E words of a thread keep the same side. A 64-bit word
// moves as two 32-bit halves.
template <int D>
__device__ __forceinline__ uint32_t lane_xor_w(uint32_t v) {
    return lane_xor<D>(v);
}
template <int D>
__device__ __forceinline__ uint64_t lane_xor_w(uint64_t v) {
    const uint32_t lo = lane_xor<D>((uint32_t)v);
    const uint32_t hi = lane_xor<D>((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}
template <int E, int D, class W>
__device__ __forceinline__ void bitonic_lane_stage(W (&v)[E], uint32_t i0, uint32_t size) {
    const bool big = keeps_larger(i0, (uint32_t)(D * E), size);
#pragma unroll
    for (int e = 0; e < E; ++e) {
        v[e] = keep_side(v[e], lane_xor_w<D>(v[e]), big);
    }
}

// Register form: n2 <= E * NT words, thread t holding words E*t .. E*t+E-1
// in v (threads past n2 / E hold padding). Within a run size, the stages go
// j = size/2 down to 1: through LDS (buf: n2 words, twice that for 32-bit
// words; between workgroup barriers) while j >= 64*E, then across the lanes
// of the wave with vector lane moves while j >= E, then inside the thread.
// Waves without a word only take part in the barriers.
template <int NW, int E, class W>
__device__ __forceinline__ void bitonic_regs(W (&v)[E], uint32_t n2, W* buf, RunState* prof = nullptr) {
    static_assert(E == 4, "in-thread stages of distance 1 and 2");
    const uint32_t i0 = threadIdx.x * E;
    const bool holds = i0 < n2;
    const bool wave_holds = (uint32_t)wave_id() * 64u * E < n2;
    if (!wave_holds && n2 <= 64u * E) return;  // no stage through LDS: nothing to join
    bool upper = false, entered = false;  // 32-bit words: the buffer half the next LDS stage uses; a stage ran
    for (uint32_t size = 2; size <= n2; size <<= 1) {
        uint32_t j = size >> 1;
        if constexpr (sizeof(W) == 4) {
            // 32-bit words: the buffer (n2 64-bit words) holds two halves of
            // n2 words, and the stages use them in turn, so one barrier per
            // stage is enough. A stage writes the half that the stage before
            // the last one read, and every wave has finished those reads
            // before it passes the last stage's barrier. The first stage
            // waits for the buffer's earlier users.
            for (; j >= 64u * E; j >>= 1) {
                W* h = buf + (upper ? n2 : 0u);
                upper = !upper;
                if (!entered) lds_barrier();
                entered = true;
                if (holds) *reinterpret_cast<u32x4*>(h + i0) = u32x4{v[0], v[1], v[2], v[3]};
                lds_barrier();
                if (holds) {
                    const bool big = keeps_larger(i0, j, size);  // the same for the thread's E words
                    const u32x4 o = *reinterpret_cast<const u32x4*>(h + (i0 ^ j));
#pragma unroll
                    for (int e = 0; e < E; ++e) v[e] = keep_side(v[e], o[e], big);
                }
            }
        }
        for (; j >= 64u * E; j >>= 1) {
            lds_barrier();  // the previous stage through LDS has been read
            if (holds) {
#pragma unroll
                for (int e = 0; e < E; ++e) buf[i0 + e] = v[e];
            }
            lds_barrier();
            if (holds) {
                const bool big = keeps_larger(i0, j, size);  // the same for the thread's E words
                W o[E];  // all reads issued before the first compare
#pragma unroll
                for (int e = 0; e < E; ++e) o[e] = buf[(i0 + e) ^ j];
#pragma unroll
                for (int e = 0; e < E; ++e) v[e] = keep_side(v[e], o[e], big);
            }
        }
#ifdef DS_PROFILE
        if (prof) prof->prof_mark(11);  // stages through LDS
#endif
        if (!wave_holds) continue;
        if (j == 32u * E) bitonic_lane_stage<E, 32>(v, i0, size), j >>= 1;
        if (j == 16u * E) bitonic_lane_stage<E, 16>(v, i0, size), j >>= 1;
        if (j == 8u * E) bitonic_lane_stage<E, 8>(v, i0, size), j >>= 1;
        if (j == 4u * E) bitonic_lane_stage<E, 4>(v, i0, size), j >>= 1;
        if (j == 2u * E) bitonic_lane_stage<E, 2>(v, i0, size), j >>= 1;
        if (j == 1u * E) bitonic_lane_stage<E, 1>(v, i0, size), j >>= 1;
#ifdef DS_PROFILE
        if (prof) prof->prof_mark(12);  // stages across lanes
#endif
        if (j == 2u) bitonic_in_thread<E, 2>(v, i0, size), j >>= 1;
        if (j == 1u) bitonic_in_thread<E, 1>(v, i0, size);
#ifdef DS_PROFILE
        if (prof) prof->prof_mark(13);  // stages inside the thread
#endif
    }
}

// Sort word of the row's result j (j < k).
template <class D>
__device__ __forceinline__ uint64_t sort_word(const Lds<D>& s, uint32_t j) {
    uint32_t key, col;
    if constexpr (is_packed<D>::value) {
        const uint32_t e = s.keys[j];
        key = e >> 16;
        col = e & 0xFFFFu;
    } else {
        key = s.keys[j];
        col = s.idx[j];
    }
    return ((uint64_t)key << 32) | (uint32_t)~col;
}

// Output entry j of a row: a result (raw bits, column), or past a short row's
// results the filler: index -1 with the bits of negative infinity.
template <class D>
__device__ __forceinline__ void put_out(const Params& p, int64_t row, uint32_t j, uint32_t raw, int32_t col) {
    const int64_t k = p.k;
    if constexpr (D::kBytes == 4)
        reinterpret_cast<uint32_t*>(p.out_vals)[row * k + j] = raw;
    else
        reinterpret_cast<uint16_t*>(p.out_vals)[row * k + j] = (uint16_t)raw;
    p.out_idx[row * k + j] = col;
}
template <class D>
__device__ __forceinline__ void put_filler(const Params& p, int64_t row, uint32_t j) {
    put_out<D>(p, row, j, D::kBytes == 4 ? 0xFF800000u : 0xFF80u, -1);
}

template <class D>
__device__ __forceinline__ void put_sorted(const Params& p, int64_t row, uint32_t j, uint64_t w, uint32_t cnt) {
    if (j < cnt)
        put_out<D>(p, row, j, D::raw((uint32_t)(w >> 32)), (int32_t)~(uint32_t)w);
    else
        put_filler<D>(p, row, j);
}

// Inclusive prefix sum over the 64 lanes of a wave, in float (the same DPP
// steps as the integer one).
__device__ __forceinline__ float wave_prefix_sum_f(float v) {
    v += __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), 0x111, 0xF, 0xF, true));
    v += __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), 0x112, 0xF, 0xF, true));
    v += __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), 0x114, 0xF, 0xF, true));
    v += __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), 0x118, 0xF, 0xF, true));
    v += __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), 0x142, 0xA, 0xF, false));
    v += __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), 0x143, 0xC, 0xF, false));
    return v;
}

template <class D>
__device__ __forceinline__ float value_of(uint32_t raw) {
    return __uint_as_float(D::kBytes == 4 ? raw : raw << 16);
}

// Fused sampling over a row's cnt results, held sorted as words v (position
// i0 + e, descending): the softmax of the values at temperature 1/inv_temp
// (the max-subtracted exponentials over their sum, as in the softmax of
// "常见CUDA手写实现"), written to probs in output order, and one draw by the
// inverse of its cumulative distribution in that order: the smallest prefix
// whose probability reaches top_p is kept, and the sample is the first
// position whose running sum of exponentials passes u times the prefix's sum.
// A row whose largest value is -inf or NaN (or that is empty) gets zero
// probabilities and sample -1; when the largest value is +inf the +inf
// results share the mass equally and the others get 0 (the limit of the
// softmax as the largest value grows). Every wave takes part (workgroup
// barriers); red is LDS scratch of NW + 4 words.
template <class D, int NW, int E>
__device__ __forceinline__ void softmax_sample(const uint64_t (&v)[E], uint32_t i0, uint32_t cnt, const Params& p,
                                               int64_t row, uint32_t* red) {
    const uint32_t k = (uint32_t)p.k;
    const int w = wave_id();
    uint32_t* r_max = red + NW;
    uint32_t* r_jp = red + NW + 1;
    uint32_t* r_cz = red + NW + 2;
    uint32_t* r_js = red + NW + 3;
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        x[e] = i0 + e < cnt ? value_of<D>(D::raw((uint32_t)(v[e] >> 32))) : -__builtin_huge_valf();
    if (threadIdx.x == 0) {
        *r_max = __float_as_uint(x[0]);
        *r_jp = ~0u;
        *r_js = ~0u;
    }
    lds_barrier();
    const float m = __uint_as_float(*r_max);
    const bool live = cnt > 0 && m > -__builtin_huge_valf();  // false for -inf and NaN
    const bool pinf = m == __builtin_huge_valf();
    float ex[E], ts = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        // NaN and -inf results add nothing (-inf > -inf and NaN > -inf are false)
        const float w = pinf ? (x[e] == __builtin_huge_valf() ? 1.f : 0.f) : expf((x[e] - m) * p.inv_temp);
        ex[e] = live && i0 + e < cnt && x[e] > -__builtin_huge_valf() ? w : 0.f;
        ts += ex[e];
    }
    const float incl = wave_prefix_sum_f(ts);
    if (lane_id() == 63) red[w] = __float_as_uint(incl);
    lds_barrier();
    float before = 0.f, Z = 0.f;  // sums of the waves before this one, and of all
#pragma unroll
    for (int q = 0; q < NW; ++q) {
        const float t = __uint_as_float(red[q]);
        before += q < w ? t : 0.f;
        Z += t;
    }
    float c[E];  // running sum of exponentials through each position
    float run = before + incl - ts;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        run += ex[e];
        c[e] = run;
        if (p.probs && i0 + e < k) p.probs[row * k + i0 + e] = live ? ex[e] / Z : 0.f;
    }
    if (!p.sample_u) return;
    // the top-p prefix: positions 0 .. jp
    uint32_t jp = cnt - 1;
    float zp = Z;
    if (p.top_p < 1.f) {
        const float lim = p.top_p * Z;
        uint32_t mine = ~0u;
#pragma unroll
        for (int e = E - 1; e >= 0; --e)
            if (i0 + e < cnt && c[e] >= lim) mine = i0 + e;
        if (mine != ~0u) atomicMin(r_jp, mine);
        lds_barrier();
        jp = *r_jp == ~0u ? cnt - 1 : *r_jp;
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (i0 + e == jp) *r_cz = __float_as_uint(c[e]);
        lds_barrier();
        zp = __uint_as_float(*r_cz);
    }
    const float target = p.sample_u[row] * zp;
    uint32_t mine = ~0u;
#pragma unroll
    for (int e = E - 1; e >= 0; --e)
        if (i0 + e <= jp && i0 + e < cnt && c[e] > target) mine = i0 + e;
    if (mine != ~0u) atomicMin(r_js, mine);
    lds_barrier();
    const uint32_t js = *r_js == ~0u ? jp : *r_js;
    if (!live) {
        if (threadIdx.x == 0) p.sample_idx[row] = -1;
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (i0 + e == js) p.sample_idx[row] = (int32_t)~(uint32_t)v[e];
    }
}

// Write the row's cnt results in descending order (then k - cnt fillers).
template <class D, int NW>
__device__ __forceinline__ void write_sorted(Lds<D>& s, const Params& p, int64_t row, uint32_t cnt) {
    constexpr int E = 4;
    uint64_t* buf = reinterpret_cast<uint64_t*>(s.base + p.L.sort);
    const uint32_t k = (uint32_t)p.k;
    const uint32_t n2 = k <= 1u ? 1u : 1u << (32 - __clz(k - 1u));
    if (n2 <= (uint32_t)(E * NW * 64)) {
#ifdef DS_PROFILE
        RunState pst;  // cycle accounting of the sort's phases only
#endif
        const uint32_t i0 = threadIdx.x * E;
        uint64_t v[E];
        uint32_t lo = 0xFFFFFFFFu, hi = 0;  // the results' smallest and largest keys
#pragma unroll
        for (int e = 0; e < E; ++e) {
            v[e] = i0 + e < cnt ? sort_word<D>(s, i0 + e) : 0ull;
            if (i0 + e < cnt) {
                const uint32_t key = (uint32_t)(v[e] >> 32);
                lo = key < lo ? key : lo;
                hi = key > hi ? key : hi;
            }
        }
        // When the keys span few enough values, key - lo and the column fit
        // one 32-bit word, (key - lo) << cb | (cmask - column) with cb the
        // bit length of N (so the second field is at least 1 and every
        // result stays above the padding 0): the same order, at half the
        // lane moves and with 32-bit compares.
        const uint32_t wlo = wave_min(lo), whi = wave_max(hi);
        if (lane_id() == 0) {
            s.misc[8 + wave_id()] = wlo;   // the final select no longer reads these
            s.misc[16 + wave_id()] = whi;
        }
        lds_barrier();
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const uint32_t a = s.misc[8 + w], b = s.misc[16 + w];
            lo = a < lo ? a : lo;
            hi = b > hi ? b : hi;
        }
        lo = uniform(lo);
        hi = uniform(hi);
        DS_PROF(pst, 7);
        const uint32_t cb = 32u - (uint32_t)__clz((uint32_t)p.n);
        const uint32_t cmask = (1u << cb) - 1u;
        const bool narrow = cnt > 0u && cb < 32u && (uint64_t)(hi - lo) < ((uint64_t)1 << (32u - cb));
        // 16-bit keys spanning more: the key's dense rank (the number of
        // distinct result keys above it, below n2) takes its place,
        // (R - rank) << cb | (cmask - column) with R = 2^rb - 1, and a table
        // in the candidate key array gives the key of each rank back. The
        // ranks come from a bitmap of the keys present (bit key - lo) and a
        // prefix count of its bits from the top, both in the sort buffer.
        const uint32_t rb = n2 > 1u ? 32u - (uint32_t)__clz(n2 - 1u) : 1u;
        const uint32_t nbw = ((hi - lo) >> 5) + 1u;  // bitmap words
        const bool ranked = D::kBits == 16 && !narrow && cnt > 0u && rb + cb <= 32u && nbw <= n2;
        if (narrow || ranked) {
            uint32_t v32[E];
            const uint32_t R = (1u << rb) - 1u;
            uint16_t* keyof = reinterpret_cast<uint16_t*>(s.keys);  // rank -> key (read above, in v)
            if (narrow) {
#pragma unroll
                for (int e = 0; e < E; ++e)
                    v32[e] = i0 + e < cnt ? (((uint32_t)(v[e] >> 32) - lo) << cb) | (cmask - ~(uint32_t)v[e]) : 0u;
            } else {
                constexpr uint32_t NT = NW * 64;
                uint32_t* bm = reinterpret_cast<uint32_t*>(buf);
                uint32_t* above = bm + nbw;  // set bits in the words past each word
                for (uint32_t j = threadIdx.x; j < nbw; j += NT) bm[j] = 0u;
                lds_barrier();
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    if (i0 + e < cnt) {
                        const uint32_t d = (uint32_t)(v[e] >> 32) - lo;
                        atomicOr(&bm[d >> 5], 1u << (d & 31u));
                    }
                }
                lds_barrier();
                // thread t counts words [t*per, t*per + per); the bits past
                // its words are the total less an inclusive prefix over the
                // threads
                const uint32_t per = (nbw + NT - 1u) / NT;
                const uint32_t w0 = threadIdx.x * per;
                uint32_t mine = 0;
                for (uint32_t j = w0; j < w0 + per && j < nbw; ++j) mine += (uint32_t)__builtin_popcount(bm[j]);
                const uint32_t incl = wave_prefix_sum(mine);
                if (lane_id() == 63) s.tot[wave_id()] = incl;
                lds_barrier();
                uint32_t before = 0, total = 0;
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    const uint32_t t = s.tot[w];
                    before += w < wave_id() ? t : 0u;
                    total += t;
                }
                uint32_t run = total - (before + incl);  // bits in the words past this thread's
                for (uint32_t j = (w0 + per < nbw ? w0 + per : nbw); j > w0; --j) {
                    above[j - 1u] = run;
                    run += (uint32_t)__builtin_popcount(bm[j - 1u]);
                }
                lds_barrier();
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    if (i0 + e < cnt) {
                        const uint32_t key = (uint32_t)(v[e] >> 32), d = key - lo;
                        const uint32_t rank =
                            above[d >> 5] + (uint32_t)__builtin_popcount((bm[d >> 5] >> (d & 31u)) >> 1);
                        keyof[rank] = (uint16_t)key;
                        v32[e] = ((R - rank) << cb) | (cmask - ~(uint32_t)v[e]);
                    } else {
                        v32[e] = 0u;
                    }
                }
            }
            DS_PROF(pst, 8);
#ifdef DS_PROFILE
            bitonic_regs<NW, E>(v32, n2, reinterpret_cast<uint32_t*>(buf), &pst);
#else
            bitonic_regs<NW, E>(v32, n2, reinterpret_cast<uint32_t*>(buf));
#endif
            if (ranked) lds_barrier();  // the rank table is complete
            DS_PROF(pst, 9);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const uint32_t key = narrow ? (v32[e] >> cb) + lo : (uint32_t)keyof[R - (v32[e] >> cb)];
                v[e] = v32[e] != 0u ? ((uint64_t)key << 32) | (uint32_t)~(cmask - (v32[e] & cmask)) : 0ull;
            }
        } else {
            DS_PROF(pst, 8);
            bitonic_regs<NW, E>(v, n2, buf);
            DS_PROF(pst, 9);
        }
        if (p.probs || p.sample_u) softmax_sample<D, NW, E>(v, i0, cnt, p, row, s.tot);
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (i0 + e < k) put_sorted<D>(p, row, i0 + e, v[e], cnt);
        DS_PROF(pst, 10);
#ifdef DS_PROFILE
        if (p.split > 1) pst.prof_flush(2048);
#endif
    } else {
        for (uint32_t j = threadIdx.x; j < n2; j += NW * 64) buf[j] = j < cnt ? sort_word<D>(s, j) : 0ull;
        bitonic_lds<NW>(buf, n2);
        for (uint32_t j = threadIdx.x; j < k; j += NW * 64) put_sorted<D>(p, row, j, buf[j], cnt);
    }
}

// A row's statistics, when asked for (thread 0 writes them).
__device__ __forceinline__ void write_stats(const Params& p, int64_t row, uint64_t W, uint64_t A, uint64_t R,
                                            uint64_t maxlen) {
    if (p.stats && threadIdx.x == 0) {
        uint64_t* o = p.stats + row * DS_STATS_PER_ROW;
        o[DS_STAT_W] = W;
        o[DS_STAT_A] = A;
        o[DS_STAT_R] = R;
        o[DS_STAT_MAX_LEN] = maxlen;
    }
}

// Write a row's results: the cnt entries of the candidate buffer (cnt = k
// unless the row's valid length is below k), then k - cnt fillers.
template <class D, int NW>
__device__ __forceinline__ void write_row(Lds<D>& s, const Params& p, int64_t row, uint32_t cnt, uint64_t W,
                                          uint64_t A, uint64_t R, uint64_t maxlen) {
    const int64_t k = p.k;
    if (p.sorted) {
        write_sorted<D, NW>(s, p, row, cnt);
    } else if (cnt < (uint32_t)k) {
        for (uint32_t j = threadIdx.x; j < (uint32_t)k; j += NW * 64) {
            if (j >= cnt) {
                put_filler<D>(p, row, j);
            } else if constexpr (is_packed<D>::value) {
                const uint32_t e = s.keys[j];
                put_out<D>(p, row, j, D::raw(e >> 16), (int32_t)(e & 0xFFFFu));
            } else {
                put_out<D>(p, row, j, D::raw((uint32_t)s.keys[j]), (int32_t)s.idx[j]);
            }
        }
    } else if constexpr (is_packed<D>::value) {
        // one part per row: the entry's column is the row's
        for (int64_t j = threadIdx.x; j < k; j += NW * 64) {
            const uint32_t e = s.keys[j];
            reinterpret_cast<uint16_t*>(p.out_vals)[row * k + j] = (uint16_t)D::raw(e >> 16);
            p.out_idx[row * k + j] = (int32_t)(e & 0xFFFFu);
        }
    } else {
    // four entries per lane with 8- and 16-byte accesses when k and the
    // output pointers allow it
    const bool vec = (k % 4) == 0 && (reinterpret_cast<uintptr_t>(p.out_vals) % 16) == 0 &&
                     (reinterpret_cast<uintptr_t>(p.out_idx) % 16) == 0;
    if (vec) {
        for (int64_t j = (int64_t)threadIdx.x * 4; j < k; j += NW * 64 * 4) {
            const u32x4 iv = *reinterpret_cast<const u32x4*>(&s.idx[j]);
            if constexpr (D::kBytes == 4) {
                const u32x4 kv = *reinterpret_cast<const u32x4*>(&s.keys[j]);
                *reinterpret_cast<u32x4*>(reinterpret_cast<uint32_t*>(p.out_vals) + row * k + j) =
                    u32x4{D::raw(kv.x), D::raw(kv.y), D::raw(kv.z), D::raw(kv.w)};
            } else {
                const uint2 kv = *reinterpret_cast<const uint2*>(&s.keys[j]);
                const uint32_t a = D::raw(kv.x & 0xFFFFu) | (D::raw(kv.x >> 16) << 16);
                const uint32_t b = D::raw(kv.y & 0xFFFFu) | (D::raw(kv.y >> 16) << 16);
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out_vals) + row * k + j) = uint2{a, b};
            }
            *reinterpret_cast<u32x4*>(p.out_idx + row * k + j) = iv;
        }
    } else {
        for (int64_t j = threadIdx.x; j < k; j += NW * 64) {
            const uint32_t key = s.keys[j];
            if constexpr (D::kBytes == 4)
                reinterpret_cast<uint32_t*>(p.out_vals)[row * k + j] = D::raw(key);
            else
                reinterpret_cast<uint16_t*>(p.out_vals)[row * k + j] = (uint16_t)D::raw(key);
            p.out_idx[row * k + j] = (int32_t)s.idx[j];
        }
    }
    }
    write_stats(p, row, W, A, R, maxlen);
}

// Part results of split rows go to the workspace for the merge kernel.
template <class D, int NW>
__device__ __forceinline__ void write_part(Lds<D>& s, const RunState& st, const Params& p, int64_t slot,
                                           uint32_t part_elem0) {
    // the part's number of results: k, or fewer for a short part or one
    // filtered by a shared threshold; its largest result key is the largest
    // key appended (that one is always kept), reduced over the waves
    const uint32_t wmax = wave_max(st.kmax);
    if (lane_id() == 0) s.misc[8 + wave_id()] = wmax;
    lds_barrier();
    if (p.ws_cnt && threadIdx.x == 0) {
        uint32_t tmax = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) tmax = s.misc[8 + w] > tmax ? s.misc[8 + w] : tmax;
        p.ws_cnt[slot] = st.len;
        p.ws_tkey[slot] = st.len == (uint32_t)p.k && st.tset ? st.tkey : 0u;
        p.ws_tmax[slot] = st.len != 0u ? tmax : 0u;
    }
    if constexpr (is_packed<D>::value) {
        // packed bfloat16 results stay one word each, key << 16 | column
        // inside the part (the merge adds the part's first column): 4 bytes
        // a result, 16-byte stores when k allows
        (void)part_elem0;
        if (p.k % 4 == 0) {
            for (int64_t j = (int64_t)threadIdx.x * 4; j < p.k; j += NW * 64 * 4)
                *reinterpret_cast<u32x4*>(p.ws_keys + slot * p.k + j) = *reinterpret_cast<const u32x4*>(&s.keys[j]);
        } else {
            for (int64_t j = threadIdx.x; j < p.k; j += NW * 64) p.ws_keys[slot * p.k + j] = s.keys[j];
        }
    } else if (p.k % 4 == 0) {  // the workspace arrays are 256-byte aligned
        for (int64_t j = (int64_t)threadIdx.x * 4; j < p.k; j += NW * 64 * 4) {
            u32x4 kv;
            if constexpr (D::kBytes == 4) {
                kv = *reinterpret_cast<const u32x4*>(&s.keys[j]);
            } else {
                const uint2 h = *reinterpret_cast<const uint2*>(&s.keys[j]);
                kv = u32x4{h.x & 0xFFFFu, h.x >> 16, h.y & 0xFFFFu, h.y >> 16};
            }
            *reinterpret_cast<u32x4*>(p.ws_keys + slot * p.k + j) = kv;
            *reinterpret_cast<u32x4*>(p.ws_idx + slot * p.k + j) = *reinterpret_cast<const u32x4*>(&s.idx[j]);
        }
    } else {
        for (int64_t j = threadIdx.x; j < p.k; j += NW * 64) {
            p.ws_keys[slot * p.k + j] = (uint32_t)s.keys[j];
            p.ws_idx[slot * p.k + j] = s.idx[j];
        }
    }
    if (threadIdx.x == 0) {
        uint64_t* o = p.ws_stats + slot * DS_STATS_PER_ROW;
        o[DS_STAT_W] = st.W;
        o[DS_STAT_A] = st.A;
        o[DS_STAT_R] = st.R;
        o[DS_STAT_MAX_LEN] = st.maxlen;
    }
}

// Valid length of a row: lengths[row] clamped to [0, n], or n.
__device__ __forceinline__ int64_t row_len(const Params& p, int64_t row) {
    if (!p.lengths) return p.n;
    const int64_t v = p.lengths[row];
    return v < 0 ? 0 : (v > p.n ? p.n : v);
}

struct PartGeom {
    int64_t row, slot, b0, part_elem0, part_n;
    int32_t part, ms;
};

__device__ __forceinline__ PartGeom part_geom(const Params& p, int64_t item) {
    PartGeom g;
    g.row = item / p.split;
    g.part = (int32_t)(item % p.split);
    g.slot = item;
    const int64_t n_r = row_len(p, g.row);
    const int64_t m = p.lengths ? ceil_div(n_r, (int64_t)p.B) : p.m;
    g.b0 = part_begin(m, g.part, p.split);
    const int64_t b1 = part_begin(m, g.part + 1, p.split);
    g.ms = (int32_t)(b1 - g.b0);
    g.part_elem0 = g.b0 * (int64_t)p.B;
    const int64_t e1 = b1 * (int64_t)p.B < n_r ? b1 * (int64_t)p.B : n_r;
    g.part_n = e1 > g.part_elem0 ? e1 - g.part_elem0 : 0;
    return g;
}

// Buffer resource over a part's elements. With kVec the range is rounded up
// to whole 16-byte loads: a row's valid length need not be a multiple of
// them, and the 16-byte path only runs on rows whose full length is (so the
// rounded range stays inside the row); the elements past the part are masked
// after the load.
template <class D, bool kVec = true>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(const Params& p, const PartGeom& g) {
    const unsigned char* rowp =
        reinterpret_cast<const unsigned char*>(p.x) + (g.row * p.row_stride + g.part_elem0) * D::kBytes;
    const int64_t v = kVec ? D::kPerLoad : 1;
    const int64_t n = (g.part_n + v - 1) / v * v;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(rowp), (short)0, (int)(n * D::kBytes),
                                             (int)kRsrcWord3);
}

template <class D, int NW, int U, int Q>
__global__ __launch_bounds__(NW * 64) void deepselect_stream_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    Lds<D> s = lds_of<D>(smem, p.L);
    const int64_t items = p.batch * (int64_t)p.split;
    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const PartGeom g = part_geom(p, item);
        lds_barrier();  // LDS free from the previous item
        begin_item<D, NW>(s);
        build_order<NW>(s.perm, p.seed, g.row, 0, g.b0, g.ms, s.base);
        RunState st;
        Streamer<D, NW, U, Q> sm{s,
                                 st,
                                 part_rsrc<D>(p, g),
                                 (uint32_t)g.part_elem0,
                                 (uint32_t)g.part_n,
                                 (uint32_t)p.B,
                                 g.ms,
                                 (int32_t)ceil_div(g.ms, NW),
                                 (uint32_t)p.k,
                                 (uint32_t)p.B2};
        sm.run();
        final_select<D, NW>(s, st, (uint32_t)p.k);
        if (p.split == 1)
            write_row<D, NW>(s, p, g.row, st.len, st.W, st.A, st.R, st.maxlen);
        else
            write_part<D, NW>(s, st, p, g.slot, (uint32_t)g.part_elem0);
    }
}

template <class D, int NW, int U>
__global__ __launch_bounds__(NW * 64) void deepselect_ring_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    Lds<D> s = lds_of<D>(smem, p.L);
    u32x4* ring = reinterpret_cast<u32x4*>(smem + p.L.ring) + (size_t)wave_id() * p.L.ring_depth * U * 64;
    const int64_t items = p.batch * (int64_t)p.split;
    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const PartGeom g = part_geom(p, item);
        lds_barrier();  // LDS free from the previous item
        RunState st;
        begin_item<D, NW>(s);
        build_order<NW>(s.perm, p.seed, g.row, 0, g.b0, g.ms, s.base);
        DS_PROF(st, 0);
        RingStreamer<D, NW, U> sm{s,
                                  st,
                                  part_rsrc<D>(p, g),
                                  (uint32_t)g.part_elem0,
                                  (uint32_t)g.part_n,
                                  (uint32_t)p.B,
                                  g.ms,
                                  (int32_t)ceil_div(g.ms, NW),
                                  p.L.ring_depth,
                                  (uint32_t)p.k,
                                  (uint32_t)p.B2,
                                  ring,
                                  p.ws_share ? p.ws_share + g.row * kCellWords : nullptr};
        sm.run();
        DS_PROF(st, 14);
        final_select<D, NW>(s, st, (uint32_t)p.k, p.ws_share != nullptr);
        DS_PROF(st, 11);
        const Params pe = reload_params();
        if (pe.split == 1)
            write_row<D, NW>(s, pe, g.row, st.len, st.W, st.A, st.R, st.maxlen);
        else
            write_part<D, NW>(s, st, pe, g.slot, (uint32_t)g.part_elem0);
        DS_PROF(st, 12);
        if constexpr (is_packed<D>::value) {
            if (pe.ws_arrive && arrive_last(pe, g.row, s.misc + 4)) merge_in_part_kernel<NW>(smem, pe, g.row);
        }
#ifdef DS_PROFILE
        st.prof_flush();
#endif
    }
}

// ===========================================================================
// Generic kernel: the whole workgroup shares each block; a tile is one 16-byte
// load (or V scalar loads) per lane, one barrier per tile. Any alignment, any N,
// any block size.
// ===========================================================================
constexpr int kGW = 4;  // waves of the generic and merge kernels

// Workgroup-cooperative append (one tile spread over all waves): wave counts
// from the ballot masks, a prefix over the waves through LDS (one barrier),
// then each survivor's slot from mbcnt. `put(slot, pos)` stores slot's element
// at buffer position pos. Returns the number appended (uniform).
template <int NW, int NS, class Put>
__device__ __forceinline__ uint32_t append_masked(const uint64_t (&masks)[NS], const bool (&pred)[NS],
                                                  uint32_t len, uint32_t* cnt, uint32_t& par, Put&& put) {
    uint32_t c = 0;
#pragma unroll
    for (int q = 0; q < NS; ++q) c += (uint32_t)__popcll(masks[q]);
    const int wave = wave_id();
    if (lane_id() == 0) cnt[par * NW + wave] = c;
    lds_barrier();
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
        for (int q = 0; q < NS; ++q) {
            if (pred[q]) put(q, off + lanes_below(masks[q]));
            off += (uint32_t)__popcll(masks[q]);
        }
    }
    return total;
}

template <class D, bool kVec>
struct TileRegs {
    u32x4 v[kVec ? 1 : (D::kPerLoad + 3) / 4];
};

template <class D, bool kVec>
__device__ __forceinline__ int tile_elem(int q) {
    if constexpr (kVec)
        return (int)threadIdx.x * D::kPerLoad + q;
    else
        return q * kGW * 64 + (int)threadIdx.x;
}

template <class D, bool kVec>
__device__ __forceinline__ void load_tile(TileRegs<D, kVec>& r, __amdgpu_buffer_rsrc_t rsrc, int64_t elem_off,
                                          int32_t tv) {
    constexpr int V = D::kPerLoad;
    if constexpr (kVec) {
        const bool ok = (int)threadIdx.x * V < tv;
        const uint32_t off = ok ? (uint32_t)((elem_off + (int64_t)threadIdx.x * V) * D::kBytes) : kOob;
        r.v[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
    } else {
#pragma unroll
        for (int q = 0; q < V; ++q) {
            const int e = tile_elem<D, kVec>(q);
            const uint32_t off = e < tv ? (uint32_t)((elem_off + e) * D::kBytes) : kOob;
            uint32_t val;
            if constexpr (D::kBytes == 4)
                val = __builtin_amdgcn_raw_buffer_load_b32(rsrc, off, 0, 0);
            else
                val = __builtin_amdgcn_raw_buffer_load_b16(rsrc, off, 0, 0);
            r.v[q / 4][q % 4] = val;
        }
    }
}

template <class D, bool kVec>
__device__ __forceinline__ uint32_t tile_raw(const TileRegs<D, kVec>& r, int q) {
    if constexpr (kVec && D::kBytes == 2) {
        const uint32_t w = r.v[0][q >> 1];
        return (q & 1) ? (w >> 16) : (w & 0xFFFFu);
    } else {
        return r.v[q / 4][q % 4];
    }
}
template <class D, bool kVec>
__device__ __forceinline__ uint32_t tile_word(const TileRegs<D, kVec>& r, int q) {
    if constexpr (D::kBytes == 4) {
        return r.v[q / 4][q % 4];
    } else if constexpr (kVec) {
        const uint32_t d = r.v[0][q >> 1];
        return (q & 1) ? d : (d << 16);
    } else {
        return r.v[q / 4][q % 4] << 16;
    }
}

template <class D, bool kVec>
__device__ __forceinline__ void generic_tile(Lds<D>& s, RunState& st, const TileRegs<D, kVec>& r, int64_t col0,
                                             int32_t tv) {
    constexpr int V = D::kPerLoad;
    if (tv <= 0) return;
    uint32_t kmax = 0;
    if (!st.fset) {
#pragma unroll
        for (int q = 0; q < V; ++q) {
            const int e = tile_elem<D, kVec>(q);
            if (e < tv) {
                const uint32_t key = D::key(tile_raw<D, kVec>(r, q));
                s.keys[st.len + (uint32_t)e] = (typename D::Key)key;
                s.idx[st.len + (uint32_t)e] = (uint32_t)(col0 + e);
                kmax = key > kmax ? key : kmax;
            }
        }
        publish_max(st, kmax);
        st.len += (uint32_t)tv;
        st.A += (uint32_t)tv;
        return;
    }
    const Thresh th = make_thresh<D>(st.fkey);
    bool pred[V];
    uint64_t masks[V];
#pragma unroll
    for (int q = 0; q < V; ++q) {
        pred[q] = tile_elem<D, kVec>(q) < tv && above(tile_word<D, kVec>(r, q), th);
        masks[q] = __ballot(pred[q]);
    }
    const uint32_t added = append_masked<kGW, V>(masks, pred, st.len, s.cnt, st.par, [&](int q, uint32_t pos) {
        const uint32_t key = D::key(tile_raw<D, kVec>(r, q));
        s.keys[pos] = (typename D::Key)key;
        s.idx[pos] = (uint32_t)(col0 + tile_elem<D, kVec>(q));
        kmax = key > kmax ? key : kmax;
    });
    publish_max(st, kmax);
    st.len += added;
    st.A += added;
}

template <class D, bool kVec, int P>
__device__ void generic_stream(Lds<D>& s, RunState& st, const Params& p, __amdgpu_buffer_rsrc_t rsrc,
                               int64_t part_elem0, int64_t part_n, int32_t ms) {
    constexpr int kTE = kGW * 64 * D::kPerLoad;
    const int64_t B = p.B;
    const int32_t tpb = (int32_t)ceil_div(B, kTE);
    const int32_t ntiles = ms * tpb;
    const uint32_t k = (uint32_t)p.k, B2 = (uint32_t)p.B2;
    auto tile_geom = [&](int32_t t, int64_t& off, int32_t& tv) {
        const int32_t bi = t / tpb, sub = t - bi * tpb;
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
    TileRegs<D, kVec> ring[P];
#pragma unroll
    for (int j = 0; j < P; ++j) {
        int64_t off;
        int32_t tv;
        tile_geom(j, off, tv);
        load_tile<D, kVec>(ring[j], rsrc, off, tv);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int32_t t0 = 0; t0 < ntiles; t0 += P) {
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const int32_t t = t0 + j;
            if (t < ntiles) {
                int64_t off;
                int32_t tv;
                tile_geom(t, off, tv);
                generic_tile<D, kVec>(s, st, ring[j], part_elem0 + off, tv);
                if (t % tpb == tpb - 1) {
                    st.maxlen = st.len > st.maxlen ? st.len : st.maxlen;
                    if (st.len >= k + B2) compact<D, kGW>(s, st, k);
                }
            }
            int64_t off;
            int32_t tv;
            tile_geom(t + P, off, tv);
            load_tile<D, kVec>(ring[j], rsrc, off, tv);
        }
    }
}

template <class D, bool kVec>
__global__ __launch_bounds__(kGW * 64) void deepselect_generic_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    Lds<D> s = lds_of<D>(smem, p.L);
    const int64_t items = p.batch * (int64_t)p.split;
    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const PartGeom g = part_geom(p, item);
        lds_barrier();
        begin_item<D, kGW>(s);
        build_order<kGW>(s.perm, p.seed, g.row, 0, g.b0, g.ms, s.base);
        RunState st;
        generic_stream<D, kVec, kVec ? 8 : 4>(s, st, p, part_rsrc<D, kVec>(p, g), g.part_elem0, g.part_n, g.ms);
        final_select<D, kGW>(s, st, (uint32_t)p.k);
        if (p.split == 1)
            write_row<D, kGW>(s, p, g.row, st.len, st.W, st.A, st.R, st.maxlen);
        else
            write_part<D, kGW>(s, st, p, g.slot, (uint32_t)g.part_elem0);
    }
}

// ===========================================================================
// Merge kernel of split rows: DeepSelect over the S part results of a row, one
// block of k candidates per part, in the random order of tag 1. A tile is kMT
// candidates per lane (lanes contiguous per load); the tile after the current
// one is loaded while the current one is appended, so the loads of a row pay
// the memory latency about once.
// ===========================================================================
constexpr int kMT = 4;

// A tile as loaded: the words are unpacked where they are used, so that the
// wait for the loads falls there (after the work placed in between), not at
// the loads. Entries past the part's k slots hold a copy of its last slot;
// every use checks an entry against the part's count first.
template <bool kPkParts>
struct MergeTile {
    uint32_t w[kMT], c[kMT];
    uint32_t col0;  // packed words: the part's first column
    __device__ __forceinline__ uint32_t key(int q) const { return kPkParts ? w[q] >> 16 : w[q]; }
    __device__ __forceinline__ uint32_t col(int q) const { return kPkParts ? col0 + (w[q] & 0xFFFFu) : c[q]; }
};

// Tile t of part `part`'s results (lanes contiguous per load). kPkParts:
// the parts wrote packed bfloat16 words, key << 16 | column inside the part,
// whose first column is added back where the column is used.
template <int NW, bool kPkParts>
__device__ __forceinline__ void load_part_tile(MergeTile<kPkParts>& t, const Params& p, int64_t row, int64_t part,
                                               uint32_t tile) {
    constexpr uint32_t TE = NW * 64 * kMT;
    const uint32_t k = (uint32_t)p.k;
    const uint32_t t0 = tile * TE;
    const int64_t off = (row * p.split + part) * (int64_t)k + t0;
    t.col0 = 0;
    if constexpr (kPkParts) {
        const int64_t m = p.lengths ? ceil_div(row_len(p, row), (int64_t)p.B) : p.m;
        t.col0 = (uint32_t)(part_begin(m, part, p.split) * p.B);
    }
    // unconditional loads at an index clamped into the part's slots (a
    // conditional load would be waited for before the next is issued)
#pragma unroll
    for (int q = 0; q < kMT; ++q) {
        const uint32_t e = (uint32_t)q * NW * 64 + (uint32_t)threadIdx.x;
        const int64_t at = off + (t0 + e < k ? e : k - 1u - t0);
        t.w[q] = p.ws_keys[at];
        if constexpr (!kPkParts) t.c[q] = p.ws_idx[at];
    }
}

// A part's results for the merge, read kBC per lane at a time with every
// load of a chunk issued before any is used: key and column of results
// e0 + j*64 + lane (j < kBC) of part `part`, zero past cnt.
constexpr int kBC = 8;
template <bool kPkParts>
struct PartChunk {
    uint32_t key[kBC], col[kBC];
    // The loads are unconditional, at an index clamped into the part's k
    // slots (in bounds whatever the count), and the values past cnt are
    // zeroed after: a conditional load would make the compiler wait for each
    // one before issuing the next.
    // keys only (the counting pass)
    __device__ __forceinline__ void load_keys(const Params& p, int64_t row, int64_t part, uint32_t e0, uint32_t cnt) {
        const uint32_t* base = p.ws_keys + (row * p.split + part) * (int64_t)p.k;
        const uint32_t lane = (uint32_t)lane_id(), last = (uint32_t)p.k - 1u;
        uint32_t w[kBC];
#pragma unroll
        for (int j = 0; j < kBC; ++j) {
            const uint32_t e = e0 + (uint32_t)j * 64u + lane;
            w[j] = base[e < last ? e : last];
        }
#pragma unroll
        for (int j = 0; j < kBC; ++j) {
            const uint32_t e = e0 + (uint32_t)j * 64u + lane;
            key[j] = e < cnt ? (kPkParts ? w[j] >> 16 : w[j]) : 0u;
        }
    }
    __device__ __forceinline__ void load(const Params& p, int64_t row, int64_t part, uint32_t e0, uint32_t cnt) {
        const int64_t off = (row * p.split + part) * (int64_t)p.k;
        uint32_t col0 = 0;
        if constexpr (kPkParts) {
            const int64_t m = p.lengths ? ceil_div(row_len(p, row), (int64_t)p.B) : p.m;
            col0 = (uint32_t)(part_begin(m, part, p.split) * p.B);
        }
        const uint32_t lane = (uint32_t)lane_id(), last = (uint32_t)p.k - 1u;
        uint32_t w[kBC], c[kBC];
#pragma unroll
        for (int j = 0; j < kBC; ++j) {
            const uint32_t e = e0 + (uint32_t)j * 64u + lane;
            const uint32_t ec = e < last ? e : last;
            w[j] = p.ws_keys[off + ec];
            if constexpr (!kPkParts) c[j] = p.ws_idx[off + ec];
        }
#pragma unroll
        for (int j = 0; j < kBC; ++j) {
            const uint32_t e = e0 + (uint32_t)j * 64u + lane;
            const bool in = e < cnt;
            if constexpr (kPkParts) {
                key[j] = in ? w[j] >> 16 : 0u;
                col[j] = col0 + (w[j] & 0xFFFFu);
            } else {
                key[j] = in ? w[j] : 0u;
                col[j] = in ? c[j] : 0u;
            }
        }
    }
};

// The merge's parts in order up to the first compaction, all at once. Until
// then T stays where it started, so every part's admitted results can be
// counted in parallel (wave w takes order positions w, w + NW, ...); a
// prefix sum over the order gives each part's place in the buffer and the
// first part after which the buffer holds k + B2 or more. The parts up to
// and including that one are appended in parallel: the buffer, A and max_len
// end exactly as the part-by-part loop leaves them. Returns that part's
// order position, or S when no part reaches it. cnt_of(part): the part's
// number of results.
template <class D, int NW, bool kPkParts, class CntOf>
__device__ __forceinline__ int32_t merge_bulk(Lds<D>& s, RunState& st, const Params& p, int64_t row, uint32_t* pcnt,
                                              CntOf&& cnt_of) {
    const int32_t S = p.split;
    const uint32_t k = (uint32_t)p.k, B2 = (uint32_t)p.B2;
    const int w = wave_id(), lane = lane_id();
    const bool filt = st.tset;
    const uint32_t thr = st.tkey;
    // the wave's parts kBP at a time, their loads issued together
    constexpr int kBP = 4;
    for (int32_t i0 = w; i0 < S; i0 += NW * kBP) {
        int64_t part[kBP];
        uint32_t cnt[kBP], c[kBP], most = 0;
#pragma unroll
        for (int b = 0; b < kBP; ++b) {
            const int32_t i = i0 + b * NW;
            part[b] = i < S ? (int64_t)uniform(s.perm[i]) : 0;
            cnt[b] = i < S ? cnt_of(part[b]) : 0u;
            c[b] = 0;
            most = cnt[b] > most ? cnt[b] : most;
        }
        for (uint32_t e0 = 0; e0 < most; e0 += 64 * kBC) {
            PartChunk<kPkParts> pc[kBP];
#pragma unroll
            for (int b = 0; b < kBP; ++b) pc[b].load_keys(p, row, part[b], e0, cnt[b]);
#pragma unroll
            for (int b = 0; b < kBP; ++b) {
#pragma unroll
                for (int j = 0; j < kBC; ++j)
                    c[b] += e0 + (uint32_t)j * 64u + (uint32_t)lane < cnt[b] && (!filt || pc[b].key[j] > thr) ? 1u : 0u;
            }
        }
#pragma unroll
        for (int b = 0; b < kBP; ++b) {
            const uint32_t t = wave_prefix_sum(c[b]);
            if (lane == 63 && i0 + b * NW < S) pcnt[i0 + b * NW] = t;
        }
    }
    lds_barrier();
    // wave 0: the exclusive prefix over the order in place, and the trigger
    if (w == 0) {
        uint32_t carry = st.len, end = 0;
        int32_t trig = S;
        for (int32_t i0 = 0; i0 < S; i0 += 64) {
            const int32_t i = i0 + lane;
            const uint32_t c = i < S ? pcnt[i] : 0u;
            const uint32_t incl = wave_prefix_sum(c);
            const uint64_t over = __ballot(i < S && carry + incl >= k + B2);
            if (i < S) pcnt[i] = carry + incl - c;
            if (trig == S && over != 0ull) {
                const int L = __builtin_ctzll(over);
                trig = i0 + L;
                end = carry + uniform(__builtin_amdgcn_readlane(incl, L));
            }
            carry += uniform(__builtin_amdgcn_readlane(incl, 63));
        }
        if (lane == 0) {
            s.misc[3] = (uint32_t)trig;
            s.misc[4] = trig == S ? carry : end;
        }
    }
    lds_barrier();
    const int32_t trig = (int32_t)uniform(s.misc[3]);
    const int32_t last = trig < S ? trig : S - 1;
    const uint32_t end = uniform(s.misc[4]);  // the length after the last part appended here
    uint32_t kmax = 0;
    for (int32_t i = w; i <= last; i += NW) {
        // a part that admits nothing is skipped (its count is the gap to the next place)
        uint32_t at = uniform(pcnt[i]);
        const uint32_t next = i < last ? uniform(pcnt[i + 1]) : end;
        if (next == at) continue;
        const int64_t part = (int64_t)uniform(s.perm[i]);
        const uint32_t cnt = cnt_of(part);
        for (uint32_t e0 = 0; e0 < cnt; e0 += 64 * kBC) {
            PartChunk<kPkParts> pc;
            pc.load(p, row, part, e0, cnt);
#pragma unroll
            for (int j = 0; j < kBC; ++j) {
                const bool pred = e0 + (uint32_t)j * 64u + (uint32_t)lane < cnt && (!filt || pc.key[j] > thr);
                const uint64_t m = __ballot(pred);
                if (pred) {
                    const uint32_t pos = at + lanes_below(m);
                    s.keys[pos] = (typename D::Key)pc.key[j];
                    s.idx[pos] = pc.col[j];
                    kmax = pc.key[j] > kmax ? pc.key[j] : kmax;
                }
                at += (uint32_t)__popcll(m);
            }
        }
    }
    publish_max(st, kmax);
    st.A += end - st.len;
    st.len = end;
    st.maxlen = end > st.maxlen ? end : st.maxlen;
    return trig;
}

// Tile number `tile` of the merge: tile tile % tpp of the part at order
// position tile / tpp.
template <int NW, bool kPkParts>
__device__ __forceinline__ void load_merge_tile(MergeTile<kPkParts>& t, const Params& p, const uint16_t* perm, int64_t row,
                                                int64_t tile, uint32_t tpp) {
    const int64_t i = tile / tpp;
    load_part_tile<NW, kPkParts>(t, p, row, (int64_t)uniform(perm[i]), (uint32_t)(tile - i * tpp));
}

// The merge of two parts of one tile each, held in registers (ca and cb
// results in the first and second part of the row's order): each thread
// keeps the results of its slots of both tiles, the radix select counts them
// there, and only the kept ones are
// stored, in output order, to the front of the candidate buffer (write_row
// copies them out). What it keeps, where each result lands
// and the statistics are those of the tile loop: the buffer order it stands
// for is (part in the row's order, wave, slot, lane), and the one compaction
// check that can trigger (after the second part) is counted as the loop
// counts it. LDS: misc[8, 32) and tot[0, 4 NW) for the exchanges, the
// histogram copies (clear on entry and on return); ends with a barrier.
template <class D, int NW, bool kPkParts>
__device__ __forceinline__ void merge_pair_regs(Lds<D>& s, RunState& st, const Params& p, int64_t row,
                                                const MergeTile<kPkParts>& ta, const MergeTile<kPkParts>& tb,
                                                uint32_t ca, uint32_t cb) {
    constexpr int E = 2 * kMT;
    const uint32_t k = (uint32_t)p.k, B2 = (uint32_t)p.B2;
    const int w = wave_id(), lane = lane_id();
    uint32_t key[E];
    uint64_t adm[E];  // the admitted results of each slot
    uint32_t c[2] = {0u, 0u}, kmax = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int q = e % kMT;
        key[e] = e < kMT ? ta.key(q) : tb.key(q);
        const bool in = (uint32_t)q * NW * 64 + threadIdx.x < (e < kMT ? ca : cb) && (!st.tset || key[e] > st.tkey);
        adm[e] = __ballot(in);
        kmax = in && key[e] > kmax ? key[e] : kmax;
        c[e / kMT] += (uint32_t)__popcll(adm[e]);
    }
    kmax = wave_max(kmax);
    if (lane == 0) {
        s.misc[8 + w] = kmax;
        s.misc[16 + w] = c[0];
        s.misc[24 + w] = c[1];
    }
    lds_barrier();
    uint32_t hi = 0, len0 = 0, len1 = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        hi = s.misc[8 + v] > hi ? s.misc[8 + v] : hi;
        len0 += s.misc[16 + v];
        len1 += s.misc[24 + v];
    }
    hi = uniform(hi);
    const uint32_t len = uniform(len0 + len1);
    // the statistics of the tile loop and the final select
    st.A += len;
    st.maxlen = len > st.maxlen ? len : st.maxlen;
    if (len >= k + B2) {
        st.R += 1;
        st.W += len + k;
    } else {
        st.W += len;
    }
    // the k-th key and the number of results equal to it that are kept
    // (with no more than k admitted, all of them are kept)
    uint32_t kth = 0, need = 0;
    const bool sel = len > k;
    if (sel) {
        const uint32_t lo = st.tset ? st.tkey : 0u;
        uint32_t base = lo, span = (hi > lo ? hi : lo) - lo, rank = k;
        int sh = span ? 32 - __clz(span) : 0;
        sh = sh > 8 ? sh - 8 : 0;
        uint32_t* hl = s.hist + (lane & (kHistCopies - 1));
        bool first = true;
        while (true) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const uint32_t u = key[e] - base;
                const bool in = ((adm[e] >> lane) & 1ull) && (first || u <= span);
                uint32_t* at = &hl[__builtin_amdgcn_ubfe(u, (uint32_t)(sh + 1), 7u) * kHistCopies];
                const uint32_t inc = 1u + __builtin_amdgcn_ubfe(u, (uint32_t)sh, 1u) * 0xFFFFu;
                atomicAdd(at, in ? inc : 0u);
            }
            first = false;
            lds_barrier();
            fold_pass<NW>(s.hist, s.fold);
            lds_barrier();
            uint32_t cnt;
            base += pick_bin(s.fold, rank, cnt) << sh;
            if (sh == 0) break;
            span = (1u << sh) - 1u;
            sh = sh > 8 ? sh - 8 : 0;
        }
        kth = base;
        need = rank;
    }
    // the kept results: every one above the k-th key and the first `need`
    // equal to it, in buffer order; per wave and part, the number above and
    // the number equal
    uint64_t gt[E], eq[E];
    uint32_t g[2] = {0u, 0u}, t[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const bool in = (adm[e] >> lane) & 1ull;
        gt[e] = sel ? __ballot(in && key[e] > kth) : adm[e];
        eq[e] = sel ? __ballot(in && key[e] == kth) : 0ull;
        g[e / kMT] += (uint32_t)__popcll(gt[e]);
        t[e / kMT] += (uint32_t)__popcll(eq[e]);
    }
    if (lane == 0) {
        s.tot[w] = g[0];
        s.tot[NW + w] = t[0];
        s.tot[2 * NW + w] = g[1];
        s.tot[3 * NW + w] = t[1];
    }
    lds_barrier();
    // the results above and equal before this wave's block of each part
    uint32_t gb[2] = {0u, 0u}, tb_[2] = {0u, 0u}, gall0 = 0, tall0 = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        const uint32_t g0 = s.tot[v], t0 = s.tot[NW + v], g1 = s.tot[2 * NW + v], t1 = s.tot[3 * NW + v];
        gall0 += g0;
        tall0 += t0;
        gb[0] += v < w ? g0 : 0u;
        tb_[0] += v < w ? t0 : 0u;
        gb[1] += v < w ? g1 : 0u;
        tb_[1] += v < w ? t1 : 0u;
    }
    gb[1] += gall0;
    tb_[1] += tall0;
    uint32_t out = 0, seen = 0;  // kept results and equal results of this block before the slot
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int a = e / kMT, q = e % kMT;
        if (q == 0) {
            out = uniform(gb[a] + (tb_[a] < need ? tb_[a] : need));
            seen = uniform(tb_[a]);
        }
        // the equal results of the slot that are kept: the first need - seen
        const uint32_t left = seen < need ? need - seen : 0u;
        const bool tie = (eq[e] >> lane) & 1ull;
        const uint64_t kt = __ballot(tie & (lanes_below(eq[e]) < left));
        const uint64_t km = gt[e] | kt;
        if ((km >> lane) & 1ull) {
            const MergeTile<kPkParts>& tt = e < kMT ? ta : tb;
            const uint32_t at = out + lanes_below(km);
            s.keys[at] = (typename D::Key)key[e];
            s.idx[at] = tt.col(q);
        }
        out += (uint32_t)__popcll(km);
        seen += (uint32_t)__popcll(eq[e]);
    }
    st.len = sel ? k : len;
    lds_barrier();  // the kept results, in output order, are visible to write_row
}

// The two-part merge run by the part that ends last (packed bfloat16 parts,
// k at most a tile; parts of rows cut short by a valid length may hold fewer
// than k results): the merge kernel's register merge on an LDS view of the
// part kernel's layout (16-bit keys in the candidate array, columns in the
// block ring, which both hold nothing the part still needs), with the same
// statistics.
template <int NW>
__device__ void merge_in_part_kernel(unsigned char* smem, const Params& p, int64_t row) {
    Lds<BF16T> m = lds_of<BF16T>(smem, p.L);
    m.idx = reinterpret_cast<uint32_t*>(smem + p.L.ring);
    uint32_t t0 = lane_id() < 2 ? p.ws_tkey[row * 2 + lane_id()] : 0u;
    uint32_t cnt = (uint32_t)p.k;
    if (p.lengths && lane_id() < 2) cnt = p.ws_cnt[row * 2 + lane_id()];
    MergeTile<true> a, b;
    load_part_tile<NW, true>(a, p, row, 0, 0);
    load_part_tile<NW, true>(b, p, row, 1, 0);
    t0 = wave_max(t0);
    RunState st;
    if (t0 != 0u) {
        st.tset = st.fset = true;
        st.tkey = st.fkey = t0 - 1u;
    }
    // the parts' order: (part 1, part 0) when part 1's hash is the smaller
    const uint64_t ctr0 = (uint64_t)(row * 2 + 1) << 32;
    const bool swap = splitmix_at(p.seed, ctr0 + 1u) < splitmix_at(p.seed, ctr0);
    const uint32_t c0 = uniform(__builtin_amdgcn_readlane(cnt, 0)), c1 = uniform(__builtin_amdgcn_readlane(cnt, 1));
    merge_pair_regs<BF16T, NW, true>(m, st, p, row, swap ? b : a, swap ? a : b, swap ? c1 : c0, swap ? c0 : c1);
    uint64_t W = st.W, A = st.A, R = st.R, maxlen = st.maxlen;
    if (p.stats) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint64_t* o = p.ws_stats + (row * 2 + q) * DS_STATS_PER_ROW;
            W += o[DS_STAT_W];
            A += o[DS_STAT_A];
            R += o[DS_STAT_R];
            maxlen = o[DS_STAT_MAX_LEN] > maxlen ? o[DS_STAT_MAX_LEN] : maxlen;
        }
    }
    write_row<BF16T, NW>(m, p, row, st.len, W, A, R, maxlen);
}

template <class D, int NW, bool kPkParts>
__global__ __launch_bounds__(NW * 64) void deepselect_merge_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    Lds<D> s = lds_of<D>(smem, p.L);
    constexpr uint32_t TE = NW * 64 * kMT;
    const uint32_t k = (uint32_t)p.k, B2 = (uint32_t)p.B2;
    const int32_t S = p.split;
    const uint32_t tpp = (k + TE - 1) / TE;  // tiles per part
    const int64_t tiles = (int64_t)S * tpp;
    // with two tiles in all (two parts of one tile each: k <= NW*256), both
    // are loaded before the order is built, which hides their latency
    const bool both = tiles == 2 && tpp == 1;
    uint32_t* pcnt = reinterpret_cast<uint32_t*>(smem + p.L.pcnt);
    for (int64_t row = blockIdx.x; row < p.batch; row += gridDim.x) {
        // The loads the row's start waits for come first, the first tiles
        // after them: a wait for a load also waits for every load issued
        // before it.
        // The parts' result counts (short or filtered parts), lane q holding
        // part q's (more than 64 parts: read where needed),
        const bool counted = p.lengths || p.ws_share;
        uint32_t part_cnt = k, part_max = 0xFFFFFFFFu;
        if (counted && S <= 64 && lane_id() < S) part_cnt = p.ws_cnt[row * S + lane_id()];
        // their largest keys (a part whose largest key is below the
        // admission bound t0 admits nothing, so its results are not read in
        // the bulk phase),
        if (!both && S <= 64 && lane_id() < S) part_max = p.ws_tmax[row * S + lane_id()];
        // and the largest k-th key of the parts that hold k results: the k-th
        // of any k elements of the row is at most the row's, so the merge
        // admits only results at or above it (T starts just below it).
        uint32_t t0 = 0;
        if (S <= 64) {
            if (lane_id() < S) t0 = p.ws_tkey[row * S + lane_id()];
        } else {
            for (int32_t q = lane_id(); q < S; q += 64) {
                const uint32_t t = p.ws_tkey[row * S + q];
                t0 = t > t0 ? t : t0;
            }
        }
        MergeTile<kPkParts> cur, nxt, pre0, pre1;
        if (both) {
            load_part_tile<NW, kPkParts>(pre0, p, row, 0, 0);
            load_part_tile<NW, kPkParts>(pre1, p, row, 1, 0);
        }
        t0 = wave_max(t0);
        // the previous row's final select has ended, so the histogram and the
        // largest-key cell are free to clear before the barrier that frees LDS
        begin_item<D, NW>(s);
        lds_barrier();
        RunState st;
        DS_PROF(st, 0);
        if (t0 != 0u) {
            st.tset = st.fset = true;
            st.tkey = st.fkey = t0 - 1u;
        }
        bool swap = false;

        if (both) {
            // two parts: the order is (part 1, part 0) exactly when part 1's
            // hash is the smaller (ties go to the lower id), so every thread
            // decides it from the two hashes, with no shared order
            const uint64_t ctr0 = (uint64_t)(row * 2 + 1) << 32;
            swap = splitmix_at(p.seed, ctr0 + 1u) < splitmix_at(p.seed, ctr0);
            cur = swap ? pre1 : pre0;
            nxt = swap ? pre0 : pre1;
        }
        // two parts of one tile, each holding k results, unsorted output: the
        // merge runs in registers (merge_pair_regs), not through the loop
        // (with sorted output too it gains 0.7 us on the sort's side and
        // costs the unsorted call 0.4 us in the compiled merge)
        const bool regs = both && !counted && !p.sorted;
        int64_t j0 = 0;          // the first tile the part-by-part loop takes
        int64_t tiles_end = regs ? 0 : tiles;  // and the end
        // At most one part that can admit results (a part admits none when
        // its largest key is below t0, or it has none): the order of the
        // parts changes neither the buffer nor the statistics, so no order
        // is built and the loop takes that part's tiles alone.
        bool single = false;
        int64_t sid = 0;
        if (!both && S <= 64) {
            const uint32_t my_cnt = counted ? part_cnt : k;
            const uint64_t live = __ballot(lane_id() < S && my_cnt != 0u && (t0 == 0u || part_max >= t0));
            single = __popcll(live) <= 1;
            sid = live != 0ull ? (int64_t)__builtin_ctzll(live) : -1;
        }
        if (single) {
            tiles_end = sid >= 0 ? (int64_t)tpp : 0;
            if (tiles_end > 0) load_part_tile<NW, kPkParts>(cur, p, row, sid, 0);
        } else if (!both) {
            build_order<NW>(s.perm, p.seed, row, 1, 0, S, s.base);
            DS_PROF(st, 1);
            // results of a part that can admit any (t0 != 0: T = t0 - 1 is set)
            const auto cnt_of = [&](int64_t part) -> uint32_t {
                if (S <= 64 && t0 != 0u && uniform(__builtin_amdgcn_readlane(part_max, (int)part)) < t0) return 0u;
                if (!counted) return k;
                return S <= 64 ? uniform(__builtin_amdgcn_readlane(part_cnt, (int)part))
                               : uniform(p.ws_cnt[row * S + part]);
            };
            const int32_t trig = merge_bulk<D, NW, kPkParts>(s, st, p, row, pcnt, cnt_of);
            DS_PROF(st, 2);
            if (trig < S) compact<D, NW>(s, st, k);
            j0 = (int64_t)(trig + 1) * tpp;
        }
        // The tile to take after tile j - 1: a whole part whose largest key
        // is at or below T admits nothing, so its tiles are not read (its
        // compaction check would repeat the one before it). Decided with T
        // as it stands when the tile is requested; a part T passes later is
        // read and filters to nothing.
        const auto next_tile = [&](int64_t j) -> int64_t {
            if (single || both || S > 64) return j;
            while (j < tiles && j % tpp == 0 && st.tset &&
                   uniform(__builtin_amdgcn_readlane(part_max, (int)uniform(s.perm[j / tpp]))) <= st.tkey)
                j += tpp;
            return j;
        };
        j0 = next_tile(j0);
        if (!single && !both && j0 < tiles) load_merge_tile<NW, kPkParts>(cur, p, s.perm, row, j0, tpp);
        for (int64_t j = j0, jn = 0; j < tiles_end; j = jn) {
            jn = next_tile(j + 1);
            if (single) {
                if (jn < tiles_end) load_part_tile<NW, kPkParts>(nxt, p, row, sid, (uint32_t)jn);
            } else if (!both && jn < tiles) {
                load_merge_tile<NW, kPkParts>(nxt, p, s.perm, row, jn, tpp);
            }
            const uint32_t t0 = (uint32_t)(j % tpp) * TE;
            // results of the part: k, or fewer for a part shorter than k or
            // one filtered by a shared threshold
            uint32_t cnt = k;
            if (counted) {
                const int64_t i = j / tpp;
                const int64_t part = single ? sid : both ? (swap ? 1 - i : i) : (int64_t)uniform(s.perm[i]);
                cnt = S <= 64 ? uniform(__builtin_amdgcn_readlane(part_cnt, (int)part))
                              : uniform(p.ws_cnt[row * S + part]);
            }
            const uint32_t tv = t0 < cnt ? ((cnt - t0) < TE ? (cnt - t0) : TE) : 0u;
            uint32_t kmax = 0;
            if (!st.tset) {
#pragma unroll
                for (int q = 0; q < kMT; ++q) {
                    const uint32_t e = (uint32_t)q * NW * 64 + (uint32_t)threadIdx.x;
                    if (e < tv) {
                        s.keys[st.len + e] = (typename D::Key)cur.key(q);
                        s.idx[st.len + e] = cur.col(q);
                        kmax = cur.key(q) > kmax ? cur.key(q) : kmax;
                    }
                }
                st.len += tv;
                st.A += tv;
            } else {
                bool pred[kMT];
                uint64_t masks[kMT];
#pragma unroll
                for (int q = 0; q < kMT; ++q) {
                    const uint32_t e = (uint32_t)q * NW * 64 + (uint32_t)threadIdx.x;
                    pred[q] = e < tv && cur.key(q) > st.tkey;
                    masks[q] = __ballot(pred[q]);
                }
                const uint32_t added =
                    append_masked<NW, kMT>(masks, pred, st.len, s.cnt, st.par, [&](int q, uint32_t pos) {
                        s.keys[pos] = (typename D::Key)cur.key(q);
                        s.idx[pos] = cur.col(q);
                        kmax = cur.key(q) > kmax ? cur.key(q) : kmax;
                    });
                st.len += added;
                st.A += added;
            }
            publish_max(st, kmax);
            if ((j + 1) % tpp == 0) {  // a part's block ends: the compaction check
                st.maxlen = st.len > st.maxlen ? st.len : st.maxlen;
                if (st.len >= k + B2) compact<D, NW>(s, st, k);
            }
            cur = nxt;
        }
        DS_PROF(st, 3);
        if (regs)
            merge_pair_regs<D, NW, kPkParts>(s, st, p, row, cur, nxt, k, k);
        else
            final_select<D, NW>(s, st, k);
        DS_PROF(st, 4);
        // the arguments of the row's end, read again (see reload_params)
        const Params pe = reload_params();
        // the parts' statistics: lane q takes parts q, q + 64, ..., then the
        // wave adds them up (only when asked for)
        uint64_t W = 0, A = 0, R = 0, maxlen = 0;
        if (pe.stats) {
            for (int32_t q = lane_id(); q < S; q += 64) {
                const uint64_t* o = pe.ws_stats + (row * S + q) * DS_STATS_PER_ROW;
                W += o[DS_STAT_W];
                A += o[DS_STAT_A];
                R += o[DS_STAT_R];
                maxlen = o[DS_STAT_MAX_LEN] > maxlen ? o[DS_STAT_MAX_LEN] : maxlen;
            }
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                W += __shfl_xor(W, d);
                A += __shfl_xor(A, d);
                R += __shfl_xor(R, d);
                const uint64_t m = __shfl_xor(maxlen, d);
                maxlen = m > maxlen ? m : maxlen;
            }
        }
        W += st.W;
        A += st.A;
        R += st.R;
        maxlen = st.maxlen > maxlen ? st.maxlen : maxlen;
        DS_PROF(st, 5);
        write_row<D, NW>(s, pe, row, st.len, W, A, R, maxlen);
        // every part of the row has ended (the part kernel came before): its
        // shared threshold cell is left zero for the next call
        if (pe.ws_share && threadIdx.x == 0) pe.ws_share[row * kCellWords] = 0u;
        DS_PROF(st, 6);
#ifdef DS_PROFILE
        st.prof_flush(2048);
#endif
    }
}

// Clear n shared threshold cells (kCellWords apart; those not known to be
// zero, before the parts start): a kernel, not a memset, so that the call
// stays capturable.
__global__ void deepselect_zero_kernel(uint64_t* p, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        p[i * kCellWords] = 0u;
        p[i * kCellWords + kArriveWord] = 0u;
    }
}

// ===========================================================================
// Host side.
// ===========================================================================

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
    const int64_t lo = std::max<int64_t>(ceil_div(m, kPermMax),
                                         ceil_div((n + B) * elem_bytes(dtype), kPartBytesMax));
    return std::max<int64_t>(lo, 1);
}

static bool split_ok(int64_t n, int64_t k, int64_t B, int64_t S) {
    const int64_t m = ceil_div(n, B);
    if (S < 1 || S > m || S > kMaxSplit) return false;
    return S == 1 || min_part_elems(n, B, S) >= k;
}

// Units (1 KiB per wave) per block on the streaming path; 0 when the block
// does not fit it (the generic kernel then runs).
static int stream_units(int dtype, int64_t B) {
    const int64_t bytes = B * elem_bytes(dtype);
    if (bytes % 16 != 0) return 0;
    const int64_t u = ceil_div(bytes, kUnitBytes);
    if (u <= 1) return 1;
    if (u <= 2) return 2;
    if (u <= 4) return 4;
    if (u <= 8) return 8;
    return 0;
}

static bool lds_fits(int dtype, int64_t n, int64_t k, int64_t B, int64_t B2, int64_t S, int waves,
                     bool sorted = false) {
    if (k + std::min<int64_t>(B, n) + B2 > ((int64_t)1 << 30)) return false;
    Layout L = make_layout(dtype, n, k, B, B2, S, waves);
    if (sorted && S == 1) L = with_sort(L, k);
    if (L.total > kLdsLimit) return false;
    if (S > 1) {
        Layout M = make_merge_layout(dtype, k, B2, S, kGW);
        if (sorted) M = with_sort(M, k);
        if (M.total > kLdsLimit) return false;
    }
    return true;
}

static int plan_split(int dtype, int64_t batch, int64_t n, int32_t k, int32_t B, int32_t B2, int32_t num_cus) {
    const int64_t lo = split_lower_bound(dtype, n, B);
    // Split when the rows fill at most half the compute units, about one
    // part per unit; no more parts than balance a part's streamed bytes with
    // the merge's S*k results (sqrt(N*size / 2k)); no part shorter than four
    // steps of 8 blocks, or two when the batch fills under a sixteenth of the
    // units (a part's fixed costs outweigh shorter ones); at most
    // kSplitPlanMax parts.
    constexpr int64_t kSplitPlanMax = 64;
    int64_t S = 1;
    if (batch > 0 && batch <= num_cus / 2) S = ceil_div(num_cus, batch);
    const double bal = std::floor(std::sqrt((double)n * elem_bytes(dtype) / (2.0 * (double)k)));
    S = std::min<int64_t>(S, std::max<int64_t>(1, (int64_t)bal));
    const int64_t min_blocks = batch <= num_cus / 16 ? 16 : 32;
    S = std::min<int64_t>(S, std::max<int64_t>(1, ceil_div(n, B) / min_blocks));
    S = std::min<int64_t>(S, kSplitPlanMax);
    S = std::max<int64_t>(S, lo);
    while (S > lo && (!split_ok(n, k, B, S) || !lds_fits(dtype, n, k, B, B2, S, kGW))) --S;
    if (!split_ok(n, k, B, S) || !lds_fits(dtype, n, k, B, B2, S, kGW)) return DS_ERR_UNSUPPORTED;
    return (int)S;
}

// Waves per workgroup of the streaming kernel: 8 while there is at most one
// workgroup per compute unit, else 4.
static int plan_waves(int64_t items, int32_t num_cus) { return items <= num_cus ? 8 : 4; }

struct DevInfo {
    int cus = 0;
    int lds = 0;
    bool known = false;
    void* scratch = nullptr;  // device address of this device's copy of `scratch`
};

// Devices are looked up in a fixed table (no host allocation on the call
// path, which the allocation-free entry point relies on).
constexpr int kMaxDevices = 64;
static std::mutex g_mu;
static DevInfo g_dev[kMaxDevices];

// Library-owned split workspaces (ds_workspace.hpp): one per (device,
// stream), and per thread for hipStreamPerThread, whose one handle names a
// different stream in every thread. The cache's lock is held from the choice
// of a workspace until the call's kernels are queued.
struct HipWsOps {
    bool per_thread(void* stream) const { return reinterpret_cast<hipStream_t>(stream) == hipStreamPerThread; }
    int sync(void* stream) const { return hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream)) != hipSuccess; }
    int release(void* ptr) const { return hipFree(ptr) != hipSuccess; }
    int allocate(void** ptr, size_t bytes) const { return hipMalloc(ptr, bytes) != hipSuccess; }
};
static HipWsOps g_ws_ops;
static WsCache<HipWsOps> g_ws;

static int device_info(int dev, DevInfo& out) {
    if (dev < 0 || dev >= kMaxDevices) return DS_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    DevInfo& d = g_dev[dev];
    if (!d.known) {
        if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return DS_ERR_HIP;
        if (hipDeviceGetAttribute(&d.lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
            return DS_ERR_HIP;
        d.known = true;
    }
    out = d;
    return DS_OK;
}

// Caller holds g_ws.mu() (until its kernels are queued).
static int library_workspace(int dev, hipStream_t stream, size_t bytes, void** out, bool** zeroed) {
    WsBuf* w = nullptr;
    if (g_ws.acquire(g_ws_ops, dev, reinterpret_cast<void*>(stream), bytes, &w) != 0) return DS_ERR_HIP;
    *out = w->ptr;
    *zeroed = &w->zeroed;
    return DS_OK;
}

template <class K>
static int launch_kernel(K kern, int64_t blocks, int threads, size_t lds, hipStream_t stream, const Params& prm) {
    if (lds > 64 * 1024) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds) != hipSuccess)
            return DS_ERR_HIP;
    }
    const int64_t grid = std::min<int64_t>(blocks, (int64_t)1 << 22);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), lds, stream, prm);
    return hipGetLastError() == hipSuccess ? DS_OK : DS_ERR_HIP;
}

// Register slots per wave: Q blocks of U 16-byte loads in flight, 32 loads
// (128 VGPRs) at most.
template <class D, int NW>
static int launch_stream(int units, const Params& prm, size_t lds, hipStream_t st, int64_t items) {
    switch (units) {
        case 1: return launch_kernel(deepselect_stream_kernel<D, NW, 1, 16>, items, NW * 64, lds, st, prm);
        case 2: return launch_kernel(deepselect_stream_kernel<D, NW, 2, 8>, items, NW * 64, lds, st, prm);
        case 4: return launch_kernel(deepselect_stream_kernel<D, NW, 4, 4>, items, NW * 64, lds, st, prm);
        case 8: return launch_kernel(deepselect_stream_kernel<D, NW, 8, 2>, items, NW * 64, lds, st, prm);
        default: return DS_ERR_UNSUPPORTED;
    }
}

template <class D, int NW>
static int launch_ring(int units, const Params& prm, size_t lds, hipStream_t st, int64_t items) {
    switch (units) {
        case 1: return launch_kernel(deepselect_ring_kernel<D, NW, 1>, items, NW * 64, lds, st, prm);
        case 2: return launch_kernel(deepselect_ring_kernel<D, NW, 2>, items, NW * 64, lds, st, prm);
        case 4: return launch_kernel(deepselect_ring_kernel<D, NW, 4>, items, NW * 64, lds, st, prm);
        case 8: return launch_kernel(deepselect_ring_kernel<D, NW, 8>, items, NW * 64, lds, st, prm);
        default: return DS_ERR_UNSUPPORTED;
    }
}

// Kernel choice: ring streaming when the ring fits, else register streaming;
// the generic kernel for rows the streaming kernels do not take.
enum KernelKind { kAuto = 0, kRing = 1, kRegs = 2, kGeneric = 3 };

// D: the part kernel's candidate type (packed bfloat16 entries only in the
// ring kernel); DM: the merge's, whose candidates carry row columns.
template <class D, class DM>
static int launch_all(KernelKind kind, int units, int waves, bool vec, Params prm, hipStream_t st, int64_t items) {
    int rc;
    const size_t lds = prm.L.total;
    if constexpr (is_packed<D>::value) {
        rc = waves == 8 ? launch_ring<D, 8>(units, prm, lds, st, items) : launch_ring<D, 4>(units, prm, lds, st, items);
    } else {
        if (kind == kRing)
            rc = waves == 8 ? launch_ring<D, 8>(units, prm, lds, st, items)
                            : launch_ring<D, 4>(units, prm, lds, st, items);
        else if (kind == kRegs)
            rc = waves == 8 ? launch_stream<D, 8>(units, prm, lds, st, items)
                            : launch_stream<D, 4>(units, prm, lds, st, items);
        else if (vec)
            rc = launch_kernel(deepselect_generic_kernel<D, true>, items, kGW * 64, lds, st, prm);
        else
            rc = launch_kernel(deepselect_generic_kernel<D, false>, items, kGW * 64, lds, st, prm);
    }
    if (rc != DS_OK || prm.split == 1 || prm.ws_arrive) return rc;
    // the merge runs on 8 waves when a part's k results need more than one
    // tile of 4 waves, or when 16 parts or more are counted at its start, and
    // the layout fits, else on 4 (measured: 8 waves are 2 us faster at
    // k = 2048, 4 waves 1 to 3.6 us faster at k = 512 with 8 parts)
    const int dtype = DM::kBytes == 4 ? DS_F32 : DS_BF16;
    Layout M8 = make_merge_layout(dtype, prm.k, prm.B2, prm.split, 8);
    if (prm.sorted) M8 = with_sort(M8, prm.k);
    if ((prm.k > kGW * 64 * kMT || prm.split >= 16) && M8.total <= kLdsLimit) {
        prm.L = M8;
        return launch_kernel(deepselect_merge_kernel<DM, 8, is_packed<D>::value>, prm.batch, 8 * 64, prm.L.total,
                             st, prm);
    }
    prm.L = make_merge_layout(dtype, prm.k, prm.B2, prm.split, kGW);
    if (prm.sorted) prm.L = with_sort(prm.L, prm.k);
    return launch_kernel(deepselect_merge_kernel<DM, kGW, is_packed<D>::value>, prm.batch, kGW * 64, prm.L.total, st,
                         prm);
}

// The split workspace of deepselect_topk_noalloc: a static device array,
// one copy per GPU the library runs on, held until the process ends. Host
// code never passes `scratch` itself to a kernel (on the host it names a
// stand-in, not device memory): it uses the address hipGetSymbolAddress gives
// for the current device, taken once per device.
// The first kCells cells (kCellWords * 8 bytes each) are the reserved
// shared-threshold cells; calls fit when the workspace they would need from
// a caller fits in the rest.
constexpr size_t kScratchBytes = (size_t)8 << 20;
constexpr size_t kScratchFree = kScratchBytes - (size_t)kCells * kCellWords * 8;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
// per device: the scratch's reserved cells have been cleared
static std::atomic<bool> g_scratch_zeroed[kMaxDevices];

static int scratch_of(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return DS_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    DevInfo& d = g_dev[dev];
    if (!d.scratch) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return DS_ERR_HIP;
        d.scratch = ptr;
    }
    *out = d.scratch;
    return DS_OK;
}

static int topk_impl(const void* x, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k, int32_t B,
                     int32_t B2, uint64_t seed, void* out_vals, int32_t* out_idx, void* stream,
                     const ds_options_t* opt, bool noalloc = false) {
    int st = validate_shape(dtype, batch, n, row_stride, k, B, B2);
    if (st != DS_OK) return st;
    if (noalloc && opt && opt->workspace) return DS_ERR_SCRATCH;
    if (batch == 0) return DS_OK;
    if (!x || !out_vals || !out_idx) return DS_ERR_NULL;
    const int es = elem_bytes(dtype);
    if (((uintptr_t)x % es) != 0) return DS_ERR_SHAPE;
    const int req_waves = opt ? opt->waves : 0;
    if (req_waves != 0 && req_waves != 4 && req_waves != 8) return DS_ERR_BLOCK;
    const int req_kernel = opt ? opt->kernel : 0;
    if (req_kernel < kAuto || req_kernel > kGeneric) return DS_ERR_BLOCK;
    const int sorted = opt ? opt->sorted : 0;
    if (sorted != 0 && sorted != 1) return DS_ERR_BLOCK;
    const int share_req = opt ? opt->share_threshold : 0;
    if (share_req != 0 && share_req != 1) return DS_ERR_BLOCK;
    // fused sampling: on sorted output, k within one register sort (4 words a
    // thread of 256)
    const bool sampling = opt && (opt->probs || opt->sample_u);
    float inv_temp = 1.f, top_p = 1.f;
    if (sampling) {
        if (!sorted) return DS_ERR_BLOCK;
        if (opt->sample_u && !opt->sample_idx) return DS_ERR_NULL;
        const float t = opt->temperature == 0.f ? 1.f : opt->temperature;
        const float tp = opt->top_p == 0.f ? 1.f : opt->top_p;
        if (!(t > 0.f) || !(t < __builtin_huge_valf()) || !(tp > 0.f && tp <= 1.f)) return DS_ERR_BLOCK;
        if (k > 1024) return DS_ERR_UNSUPPORTED;
        inv_temp = 1.f / t;
        top_p = tp;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DS_ERR_HIP;
    DevInfo di;
    if ((st = device_info(dev, di)) != DS_OK) return st;

    int64_t S = (opt && opt->split > 0) ? opt->split : 0;
    if (S == 0) {
        const int ps = plan_split(dtype, batch, n, k, B, B2, di.cus);
        if (ps < 0) return ps;
        S = ps;
    } else if (!split_ok(n, k, B, S) || S < split_lower_bound(dtype, n, B)) {
        return DS_ERR_BLOCK;
    }
    const bool vec = ((uintptr_t)x % 16 == 0) && ((row_stride * es) % 16 == 0) && (((int64_t)B * es) % 16 == 0) &&
                     ((n * es) % 16 == 0);
    const int units = vec ? stream_units(dtype, B) : 0;
    KernelKind kind = units > 0 ? kAuto : kGeneric;
    if (req_kernel == kGeneric) kind = kGeneric;
    int waves = kind != kGeneric ? (req_waves ? req_waves : plan_waves(batch * S, di.cus)) : kGW;
    if (!lds_fits(dtype, n, k, B, B2, S, waves, sorted)) {
        if (waves != kGW && lds_fits(dtype, n, k, B, B2, S, kGW, sorted))
            waves = kGW;
        else
            return DS_ERR_UNSUPPORTED;
    }
    // the rows' own kernel sorts its results when it writes the output (one
    // part per row; rows of two parts merged by their last part, below)
    const bool sort_here = sorted && S == 1;
    Layout L = make_layout(dtype, n, k, B, B2, S, waves);
    if (sort_here) L = with_sort(L, k);
    if ((int64_t)L.total > (int64_t)di.lds) return DS_ERR_UNSUPPORTED;
    bool packed = false;  // the ring kernel on packed bfloat16 entries
    bool pair_sorts = false;  // the part kernel's layout has room to sort a merged row
    if (kind != kGeneric) {
        const bool pk = packed_parts(dtype, n, B, S);
        Layout LB = L;
        if (pk) {
            LB = make_layout(dtype, n, k, B, B2, S, waves, true);
            if (sort_here) LB = with_sort(LB, k);
        }
        Layout LR = with_ring(LB, ceil_div(ceil_div(ceil_div(n, B), S), waves), units, (size_t)di.lds);
        // sorted rows of two packed parts that the part ending last may merge:
        // room for the sort as well, when the ring keeps its depth
        if (sorted && S == 2 && pk && !sampling && !share_req &&
            (int64_t)k <= (int64_t)waves * 64 * 4 && LR.ring_depth > 0) {
            const Layout LS =
                with_ring(with_sort(LB, k), ceil_div(ceil_div(ceil_div(n, B), S), waves), units, (size_t)di.lds);
            if (LS.ring_depth == LR.ring_depth) {
                LR = LS;
                pair_sorts = true;
            }
        }
        if (req_kernel == kRing && LR.ring_depth == 0) return DS_ERR_UNSUPPORTED;
        if (req_kernel == kRegs || LR.ring_depth == 0) {
            kind = kRegs;
        } else {
            kind = kRing;
            L = LR;
            packed = pk;
        }
    }

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
    prm.sorted = sorted;
    prm.lengths = opt ? opt->lengths : nullptr;
    prm.probs = sampling ? opt->probs : nullptr;
    prm.sample_u = sampling ? opt->sample_u : nullptr;
    prm.sample_idx = sampling ? opt->sample_idx : nullptr;
    prm.inv_temp = inv_temp;
    prm.top_p = top_p;
    prm.L = L;
    // Shared thresholds act in the ring kernel only, and from about the
    // fourth step of a wave on (a published T reaches the other parts' filter
    // two steps after it goes out): parts with fewer steps run as without it.
    const bool share = share_req && S > 1 && kind == kRing &&
                       ceil_div(ceil_div(ceil_div(n, B), S), waves) >= kShareMinSteps;
    // Rows of two packed bfloat16 parts whose k results fit one merge tile
    // (no sampling, no shared thresholds): the part that ends last merges the
    // row (an arrival count per row in its cell) and writes it, sorted when
    // asked for; no merge kernel.
    const bool fuse = S == 2 && kind == kRing && packed && (int64_t)k <= (int64_t)waves * 64 * 4 &&
                      (!sorted || pair_sorts) && !sampling && !share;

    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    std::unique_lock<std::mutex> ws_lock;  // held while a library workspace is in use
    // Shared-threshold cells: the merge leaves every cell of its rows zero, so
    // the kCells cells reserved at the start of a library workspace or of the
    // scratch (which no other array of any call overlaps) stay zero from one
    // call to the next once they have been cleared. A call clears what it
    // cannot know to be zero: all its cells in a caller workspace; the
    // reserved cells until an eager (not captured) clear has been queued;
    // cells past the reserved ones.
    bool* ws_zeroed = nullptr;                    // library workspace (under g_ws.mu())
    std::atomic<bool>* sc_zeroed = nullptr;       // scratch
    int64_t clear0 = 0, clear1 = 0;               // cells [clear0, clear1) to clear
    bool eager_clear = false;                     // the reserved cells are cleared by this call, eagerly
    uint64_t* cells = nullptr;                    // the rows' cells
    if (S > 1) {
        const bool own = noalloc || !(opt && opt->workspace);
        const WsLayout wl = make_ws_layout(batch, k, S, own ? kCells : 0);
        void* ws = nullptr;
        if (noalloc) {
            if (make_ws_layout(batch, k, S).total > kScratchFree) return DS_ERR_SCRATCH;
            if ((st = scratch_of(dev, &ws)) != DS_OK) return st;
            sc_zeroed = &g_scratch_zeroed[dev];
        } else if (!own) {
            if (opt->workspace_bytes < wl.total) return DS_ERR_WORKSPACE;
            ws = opt->workspace;
        } else {
            ws_lock = std::unique_lock<std::mutex>(g_ws.mu());
            if ((st = library_workspace(dev, hs, wl.total, &ws, &ws_zeroed)) != DS_OK) return st;
        }
        if (share || fuse) {
            clear1 = batch;
            if (own) {
                const bool zeroed = ws_zeroed ? *ws_zeroed : sc_zeroed->load();
                if (zeroed) {
                    clear0 = std::min<int64_t>(batch, kCells);
                } else {
                    clear1 = std::max<int64_t>(batch, kCells);
                    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
                    eager_clear = hipStreamIsCapturing(hs, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone;
                }
            }
        }
        unsigned char* w = reinterpret_cast<unsigned char*>(ws);
        prm.ws_keys = reinterpret_cast<uint32_t*>(w + wl.keys);
        prm.ws_idx = reinterpret_cast<uint32_t*>(w + wl.idx);
        prm.ws_stats = reinterpret_cast<uint64_t*>(w + wl.stats);
        prm.ws_cnt = reinterpret_cast<uint32_t*>(w + wl.cnt);
        prm.ws_tkey = reinterpret_cast<uint32_t*>(w + wl.tkey);
        prm.ws_tmax = reinterpret_cast<uint32_t*>(w + wl.tmax);
        cells = reinterpret_cast<uint64_t*>(w + wl.share);
        prm.ws_share = share ? cells : nullptr;
        prm.ws_arrive = fuse ? cells + kArriveWord : nullptr;
    }
    const int64_t items = batch * S;
    if (clear1 > clear0) {
        const int64_t blocks = std::min<int64_t>(ceil_div(clear1 - clear0, 256), 1024);
        hipLaunchKernelGGL(deepselect_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, hs,
                           cells + clear0 * kCellWords, clear1 - clear0);
        if (hipGetLastError() != hipSuccess) return DS_ERR_HIP;
    }
    int rc;
    if (dtype == DS_F32)
        rc = launch_all<F32T, F32T>(kind, units, waves, vec, prm, hs, items);
    else if (packed)
        rc = launch_all<BF16P, BF16T>(kind, units, waves, vec, prm, hs, items);
    else
        rc = launch_all<BF16T, BF16T>(kind, units, waves, vec, prm, hs, items);
    if (prm.ws_share || prm.ws_arrive) {
        // a failed launch may leave a part kernel's cells without their merge
        const bool zeroed = rc == DS_OK && (eager_clear || (ws_zeroed ? *ws_zeroed : sc_zeroed && sc_zeroed->load()));
        if (ws_zeroed) *ws_zeroed = zeroed;
        if (sc_zeroed) sc_zeroed->store(zeroed);
    }
    return rc;
}

}  // namespace ds

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

int deepselect_validate(int dtype, int64_t batch, int64_t N, int64_t row_stride, int32_t k, int32_t B,
                        int32_t B2) {
    const int st = ds::validate_shape(dtype, batch, N, row_stride, k, B, B2);
    if (st != DS_OK) return st;
    const int64_t lo = ds::split_lower_bound(dtype, N, B);
    if (!ds::split_ok(N, k, B, lo)) return DS_ERR_UNSUPPORTED;
    return ds::lds_fits(dtype, N, k, B, B2, lo, ds::kGW) ? DS_OK : DS_ERR_UNSUPPORTED;
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

int deepselect_topk_noalloc(const void* x, int dtype, int64_t batch, int64_t N, int64_t row_stride, int32_t k,
                            int32_t B, int32_t B2, uint64_t seed, void* out_vals, int32_t* out_idx, void* stream,
                            const ds_options_t* opt) {
    try {
        return ds::topk_impl(x, dtype, batch, N, row_stride, k, B, B2, seed, out_vals, out_idx, stream, opt, true);
    } catch (...) {
        return DS_ERR_HIP;
    }
}

size_t deepselect_scratch_bytes(void) { return ds::kScratchFree; }

#ifdef DS_PROFILE
// Profiling builds only: copy out (and clear) the per-wave cycle counts.
int ds_prof_read(void* host, size_t bytes, int clear) {
    if (hipDeviceSynchronize() != hipSuccess) return DS_ERR_HIP;
    if (hipMemcpyFromSymbol(host, HIP_SYMBOL(ds::ds_prof), bytes) != hipSuccess) return DS_ERR_HIP;
    void* p = nullptr;
    if (clear && (hipGetSymbolAddress(&p, HIP_SYMBOL(ds::ds_prof)) != hipSuccess ||
                  hipMemset(p, 0, sizeof(ds::ds_prof)) != hipSuccess))
        return DS_ERR_HIP;
    return hipDeviceSynchronize() == hipSuccess ? DS_OK : DS_ERR_HIP;
}
#endif

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
    return ds::make_layout(dtype, N, k, B, B2, split, ds::kGW).total;
}

const char* deepselect_status_string(int status) {
    switch (status) {
        case DS_OK: return "ok";
        case DS_ERR_NULL: return "a required pointer is NULL";
        case DS_ERR_DTYPE: return "dtype must be DS_F32 or DS_BF16";
        case DS_ERR_SHAPE: return "bad shape: need batch >= 0, 1 <= N < 2^31, row_stride >= N, aligned x";
        case DS_ERR_K: return "k must satisfy 1 <= k <= N";
        case DS_ERR_BLOCK:
            return "B and B2 must be >= 1; a forced split must leave every part >= k elements; waves 0, 4 or 8";
        case DS_ERR_UNSUPPORTED: return "candidate buffer k+B+B2 (or the block order) does not fit in LDS";
        case DS_ERR_HIP: return "a HIP call failed";
        case DS_ERR_WORKSPACE: return "caller workspace is smaller than deepselect_workspace_bytes";
        case DS_ERR_SCRATCH:
            return "the call needs more split workspace than the static scratch holds (deepselect_scratch_bytes), "
                   "or a workspace was passed to the allocation-free entry point";
        default: return "unknown status";
    }
}

void deepselect_release(void) { ds::g_ws.release_all(ds::g_ws_ops); }

}  // extern "C"
