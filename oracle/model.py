"""DeepSelect method model -- TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

A plain numpy run of the DeepSelect procedure of the DeepSelect deep-dive
(PFCCLab/DeepSelect, section "算法", the DeepSelectTopk pseudo-code), kept in
the page's order and notation and instrumented with the quantities of its
section "RadixSelectTopK 总处理元素数的期望上界":

* W -- total input length of all RadixSelectTopK calls, the final call included;
* A -- number of elements appended to topk_candidate;
* R -- number of RadixSelectTopK calls inside the loop (compactions);
* max_len -- largest len(topk_candidate) reached;
* the sequence of thresholds T and a per-element read count.

It does not compute the output by the same route as the oracle: the oracle
sorts, the model filters and radix-selects. The two cross-check each other.

Readings of points the pages leave open (each one is also listed in the design doc):

* Before the first compaction every element is admitted (the page states this
  outright after the pseudo-code); T is "unset" until then rather than the
  float -inf, so rows holding -inf still fill the buffer.
* Values are compared through the order-preserving key of "CUDA 算子笔记 4"
  section "改造 Radix Sort" (``oracle.keys``); x > T means key(x) > key(T).
* RadixSelectTopK is the MSD radix select of "CUDA 算子笔记 4" section
  "改造 Radix Sort": 8-bit digits from the top (4 passes for 32-bit keys, 2
  for 16-bit keys), each pass a 256-bin histogram of the keys that match the
  prefix chosen so far, then the digit that holds the k-th largest. It keeps
  every key above the k-th and the first ties equal to it, in buffer order.
* The random block order p is a permutation independent of x: the block ids
  sorted by (h, id), h the SplitMix64 output (Steele, Lea and Flood, "Fast
  splittable pseudorandom number generators", OOPSLA 2014) with counter
  ((row*2 + tag) << 32) + id, tag 0 for row blocks and 1 for the merge.
* The compaction check runs after every block, as in the pseudo-code.
* Split rows (the page's "实现" section, last paragraph: a row cut into parts,
  each part's top-k gathered and reduced to the row's top-k): part s of S owns
  the contiguous blocks [s*m//S, (s+1)*m//S) and runs DeepSelect on them; the
  merge runs DeepSelect again with one block per part (its k results), in the
  random order of tag 1, and the same k and B2, with T starting just below the
  largest k-th key among the parts that hold k results (a part's k-th never
  exceeds the row's, so nothing below it can be among the row's top k).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from oracle import BF16, F32, keys as key_of, raw_bits

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
MIX_M1 = np.uint64(0xBF58476D1CE4E5B9)
MIX_M2 = np.uint64(0x94D049BB133111EB)


# ---------------------------------------------------------------------------
# Building blocks from "并行算法（一）" (elainafan.one): scan and compact.
# ---------------------------------------------------------------------------

def inclusive_scan(a: np.ndarray) -> np.ndarray:
    """Section "Scan": out[i] = a[0] + ... + a[i]."""
    return np.cumsum(np.asarray(a, dtype=np.int64))


def exclusive_scan(a: np.ndarray) -> np.ndarray:
    """Section "Scan": out[i] = a[0] + ... + a[i-1], out[0] = 0."""
    a = np.asarray(a, dtype=np.int64)
    out = np.zeros_like(a)
    if len(a) > 1:
        out[1:] = np.cumsum(a)[:-1]
    return out


def compact(values: np.ndarray, pred: np.ndarray) -> np.ndarray:
    """Section "Compact": predicate, exclusive scan of it, scatter to the scan slot.

    The output length is the last scan value plus the last predicate.
    """
    pred = np.asarray(pred, dtype=np.int64)
    if len(pred) == 0:
        return values[:0].copy()
    s = exclusive_scan(pred)
    out = np.empty(int(s[-1] + pred[-1]), dtype=values.dtype)
    keep = pred.astype(bool)
    out[s[keep]] = values[keep]
    return out


# ---------------------------------------------------------------------------
# Random block order.
# ---------------------------------------------------------------------------

def splitmix64(seed: int, counter: np.ndarray) -> np.ndarray:
    """Output number ``counter`` (0-based) of SplitMix64 seeded with ``seed``.

    SplitMix64 adds the golden gamma 0x9E3779B97F4A7C15 to its state once per
    output and returns the mix of the new state: z ^= z >> 30, z *= M1;
    z ^= z >> 27, z *= M2; z ^= z >> 31 (all modulo 2^64).
    """
    c = np.asarray(counter, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + (c + np.uint64(1)) * GOLDEN_GAMMA
        z = (z ^ (z >> np.uint64(30))) * MIX_M1
        z = (z ^ (z >> np.uint64(27))) * MIX_M2
        z = z ^ (z >> np.uint64(31))
    return z


def block_order(seed: int, row: int, tag: int, ids: np.ndarray) -> np.ndarray:
    """The ids sorted by (SplitMix64 hash, id): a random permutation independent of x."""
    ids = np.asarray(ids, dtype=np.int64)
    ctr = (np.uint64(((row * 2 + tag) << 32) & 0xFFFFFFFFFFFFFFFF)
           + ids.astype(np.uint64))
    h = splitmix64(seed, ctr)
    return ids[np.lexsort((ids, h))]


# ---------------------------------------------------------------------------
# RadixSelectTopK ("CUDA 算子笔记 4", section "改造 Radix Sort").
# ---------------------------------------------------------------------------

def radix_select_topk(ck: np.ndarray, ci: np.ndarray, k: int, bits: int):
    """Keep the k largest keys of the candidate list; return (keys, idx, kth).

    MSD select: for each 8-bit digit from the top, histogram the digits of the
    keys that match the prefix fixed so far, walk the 256 bins from the top
    down to the one holding the rank-th largest, fix that digit and lower the
    rank by the count above it. The prefix after the last digit is the k-th
    largest key; all larger keys are kept and the first ``rank`` equal keys in
    buffer order. With len <= k everything is kept and kth is the smallest key.
    """
    n = len(ck)
    if n == 0:
        return ck, ci, None
    if n <= k:
        return ck, ci, int(ck.min())
    prefix, pmask, rank = 0, 0, k
    for shift in range(bits - 8, -1, -8):
        match = (ck & np.uint32(pmask)) == np.uint32(prefix)
        hist = np.bincount((ck[match] >> np.uint32(shift)) & np.uint32(0xFF), minlength=256)
        above = 0
        d = 255
        while above + int(hist[d]) < rank:
            above += int(hist[d])
            d -= 1
        rank -= above
        prefix |= d << shift
        pmask |= 0xFF << shift
    kth = np.uint32(prefix)
    gt = ck > kth
    tie = ck == kth
    tie_before = exclusive_scan(tie)
    sel = gt | (tie & (tie_before < rank))
    assert int(sel.sum()) == k
    return compact(ck, sel), compact(ci, sel), int(prefix)


# ---------------------------------------------------------------------------
# DeepSelectTopk.
# ---------------------------------------------------------------------------

@dataclass
class RunStats:
    W: int = 0
    A: int = 0
    R: int = 0
    max_len: int = 0
    thresholds: list = field(default_factory=list)
    all_admitted_before_first_compaction: bool = True
    selected: bool = False  # some RadixSelectTopK call had more than k entries (T was set)

    def add(self, o: "RunStats"):
        self.W += o.W
        self.A += o.A
        self.R += o.R
        self.max_len = max(self.max_len, o.max_len)
        self.thresholds += o.thresholds
        self.all_admitted_before_first_compaction &= o.all_admitted_before_first_compaction


def deepselect(blocks, k: int, block2: int, bits: int, t0=None):
    """DeepSelectTopk over ``blocks`` (a list of (keys, idx) already in scan order).

    Returns (keys, idx, kth, stats). The loop follows the pseudo-code: filter
    each block against T (everything admitted while T is unset), append the
    survivors, and compact with RadixSelectTopK whenever len >= k + B2; at the
    end RadixSelectTopK once more. ``t0``: a key every wanted result is known
    to reach; T then starts just below it (keys >= t0 are admitted from the
    first block) instead of unset.
    """
    st = RunStats()
    ck = np.empty(0, dtype=np.uint32)
    ci = np.empty(0, dtype=np.int64)
    T = None if not t0 else int(t0) - 1
    for bk, bi in blocks:
        if T is None:
            pred = np.ones(len(bk), dtype=bool)
        else:
            pred = bk > np.uint32(T)
        sk, si = compact(bk, pred), compact(bi, pred)
        if T is None and len(sk) != len(bk):
            st.all_admitted_before_first_compaction = False
        ck = np.concatenate([ck, sk])
        ci = np.concatenate([ci, si])
        st.A += len(sk)
        st.max_len = max(st.max_len, len(ck))
        if len(ck) >= k + block2:
            st.W += len(ck)
            st.R += 1
            ck, ci, T = radix_select_topk(ck, ci, k, bits)
            st.thresholds.append(T)
            st.selected = True
    st.W += len(ck)
    st.selected |= len(ck) > k
    ck, ci, kth = radix_select_topk(ck, ci, k, bits)
    return ck, ci, kth, st


@dataclass
class RowResult:
    vals: np.ndarray  # raw patterns of the k results
    idx: np.ndarray  # int64 columns
    kth: int  # k-th largest key of the row
    stats: RunStats
    reads: np.ndarray  # per-element read count


def part_bounds(m: int, split: int):
    """Block ranges [s*m//S, (s+1)*m//S) of the S parts of a row."""
    return [(s * m // split, (s + 1) * m // split) for s in range(split)]


def row_topk(x_row: np.ndarray, k: int, block: int, block2: int, seed: int = 0, row: int = 0,
             split: int = 1, length: int | None = None) -> RowResult:
    """DeepSelect on one row (float32 values or raw bfloat16 bits), S parts plus merge.

    ``length``: the row's valid length (clamped to [0, N]). The method then
    runs on the prefix x_row[:length] as on a row of that many elements: its
    blocks cut into ``split`` parts (some may hold fewer than k elements, or
    none), each part's result, and the merge over the parts' results. With
    fewer than k valid elements every one of them is returned.
    """
    raw, dt = raw_bits(np.asarray(x_row))
    bits = 32 if dt == F32 else 16
    if length is not None:
        raw = raw[:min(max(int(length), 0), len(raw))]
    keys = key_of(raw)
    n = len(keys)
    if not (k >= 1 and block >= 1 and block2 >= 1):
        raise ValueError("DeepSelectTopk requires k >= 1, B >= 1, B2 >= 1")
    if length is None and k > n:
        raise ValueError("DeepSelectTopk requires k <= N")
    m = -(-n // block)
    if split < 1 or (length is None and split > m):
        raise ValueError("split must be in [1, ceil(N/B)]")
    reads = np.zeros(n, dtype=np.int64)
    total = RunStats()
    parts = []
    for b0, b1 in part_bounds(m, split):
        blocks = []
        for b in block_order(seed, row, 0, np.arange(b0, b1)):
            lo, hi = int(b) * block, min((int(b) + 1) * block, n)
            reads[lo:hi] += 1
            blocks.append((keys[lo:hi], np.arange(lo, hi, dtype=np.int64)))
        ck, ci, kth, st = deepselect(blocks, k, block2, bits)
        total.add(st)
        parts.append((ck, ci, kth if len(ck) == k and st.selected else None))
    if split > 1:
        # the k-th largest of any k elements of the row is at most the row's,
        # so the merge admits only results at or above the largest k-th of the
        # parts that hold k (those where a select ran and set T)
        t0 = max([t for _, _, t in parts if t is not None], default=None)
        order = block_order(seed, row, 1, np.arange(split))
        ck, ci, kth, st = deepselect([parts[int(p)][:2] for p in order], k, block2, bits, t0)
        total.add(st)
    vals = raw[ci]
    return RowResult(vals=vals, idx=ci, kth=kth, stats=total, reads=reads)


def expected_w_bound(n: int, k: int, block: int, block2: int) -> float:
    """E[W] <= (1 + k/B2) * L * H_m with m = ceil(N/B), L = k+B+B2 (analysis section)."""
    m = -(-n // block)
    harmonic = math.fsum(1.0 / i for i in range(1, m + 1))
    return (1.0 + k / block2) * (k + block + block2) * harmonic


def expected_w_bound_row(n: int, k: int, block: int, block2: int, split: int = 1) -> float:
    """The bound summed over a row cut into ``split`` parts (reading c12):
    every part is a DeepSelect on its own blocks [s*m//S, (s+1)*m//S), so it
    has the boxed bound with its own m_s (its element count over B, rounded
    up), and the merge is a DeepSelect over S blocks of k results (block
    length k, the same k and B2)."""
    if split <= 1:
        return expected_w_bound(n, k, block, block2)
    m = -(-n // block)
    total = 0.0
    for b0, b1 in part_bounds(m, split):
        n_s = min(b1 * block, n) - b0 * block
        total += expected_w_bound(n_s, k, block, block2)
    return total + expected_w_bound(split * k, k, k, block2)


def batch_topk(x: np.ndarray, k: int, block: int, block2: int, seed: int = 0, split: int = 1,
               row0: int = 0, lengths=None):
    """Model over every row of ``x``; ``row0`` is the row number of x[0] (block order)."""
    out = [row_topk(x[i], k, block, block2, seed, row0 + i, split,
                    None if lengths is None else int(lengths[i])) for i in range(x.shape[0])]
    return out


__all__ = ["inclusive_scan", "exclusive_scan", "compact", "splitmix64", "block_order",
           "radix_select_topk", "deepselect", "row_topk", "batch_topk", "expected_w_bound", "expected_w_bound_row",
           "part_bounds", "RunStats", "RowResult", "F32", "BF16"]
