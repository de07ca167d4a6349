"""Pins of the DeepSelect method model (``oracle/model.py``).

The model is checked against the oracle's plain definition, the pages' worked
examples for its building blocks, the invariants and identities the
DeepSelect deep-dive states, and the expected-work bound of its analysis.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle import model

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    return json.load(open(os.path.join(GOLDEN, name)))


# ---------------------------------------------------------------- building blocks

def test_scan_worked_example():
    g = _load("scan_example.json")
    assert model.inclusive_scan(g["input"]).tolist() == g["inclusive"]
    assert model.exclusive_scan(g["input"]).tolist() == g["exclusive"]


def test_compact_worked_example():
    g = _load("compact_example.json")
    assert model.exclusive_scan(g["predicate"]).tolist() == g["exclusive_scan"]
    out = model.compact(np.array(g["input"]), np.array(g["predicate"]))
    assert out.tolist() == g["output"]


def test_splitmix64_known_answer():
    g = _load("splitmix64_seed0.json")
    got = model.splitmix64(g["seed"], np.arange(3, dtype=np.uint64))
    assert [int(v) for v in got] == [int(h, 16) for h in g["outputs_hex"]]


def test_splitmix64_outputs_of_distinct_counters_differ():
    # the state steps by an odd constant and every step of the mix is a
    # bijection of 64-bit words, so no two counters share an output: the
    # block order never needs its id tie-break (the kernels rank ids by their
    # hash alone); checked on a row's counter range for a few seeds and rows
    for seed in (0, 1, 0xDEADBEEF, 2**64 - 1):
        for row, tag in ((0, 0), (127, 1), (2**20, 0)):
            ctr = np.uint64((row * 2 + tag) << 32) + np.arange(1 << 16, dtype=np.uint64)
            h = model.splitmix64(seed, ctr)
            assert len(np.unique(h)) == h.size
    # and each mixing step inverts: z ^ (z >> s) is undone by the same
    # shifts repeated, a product by an odd constant by its inverse mod 2^64
    rng = np.random.default_rng(5)
    z = rng.integers(0, 2**63, 1000, dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    for s_ in (30, 27, 31):
        y = z ^ (z >> np.uint64(s_))
        back = y.copy()
        for _ in range(64 // s_ + 1):
            back = y ^ (back >> np.uint64(s_))
        assert np.array_equal(back, z)
    for m in (model.MIX_M1, model.MIX_M2, model.GOLDEN_GAMMA):
        inv = pow(int(m), -1, 2**64)
        with np.errstate(over="ignore"):
            assert np.array_equal(z * np.uint64(m) * np.uint64(inv), z)


def test_radix_select_against_sorting():
    rng = np.random.default_rng(1)
    for bits in (16, 32):
        for n, k in ((1, 1), (10, 3), (1000, 1), (1000, 999), (5000, 700)):
            hi = 1 << bits
            ck = rng.integers(0, hi, n, dtype=np.uint64).astype(np.uint32)
            if n > 10:
                ck[: n // 3] = ck[0]  # force heavy ties
            ci = np.arange(n)
            kk, ki, kth = model.radix_select_topk(ck, ci, k, bits)
            expect = np.sort(ck)[::-1][:k]
            assert np.array_equal(np.sort(kk)[::-1], expect)
            assert kth == int(expect[-1])
            assert np.array_equal(ck[ki], kk)
            # ties equal to the k-th are the earliest ones in buffer order
            tie_pos = np.flatnonzero(ck == kth)
            kept = np.sort(ki[kk == kth])
            assert np.array_equal(kept, tie_pos[: len(kept)])


# ---------------------------------------------------------------- block order

def test_block_order_is_a_permutation():
    for m in (1, 2, 7, 64, 149, 1024):
        for seed in (0, 1, 123456789):
            p = model.block_order(seed, 3, 0, np.arange(10, 10 + m))
            assert sorted(p.tolist()) == list(range(10, 10 + m))


def test_block_order_is_uniform():
    """Chi-square test of the position of each block over many seeds."""
    m = 8
    counts = np.zeros((m, m))
    trials = 20000
    for seed in range(trials):
        p = model.block_order(seed, 0, 0, np.arange(m))
        counts[np.arange(m), p] += 1
    expected = trials / m
    chi2 = ((counts - expected) ** 2 / expected).sum()
    # (m-1)^2 = 49 degrees of freedom; 99.9th percentile is about 85
    assert chi2 < 85.0
    # and all m! orders occur for a small m
    seen = {tuple(model.block_order(s, 1, 0, np.arange(4)).tolist()) for s in range(2000)}
    assert len(seen) == 24


def test_block_order_depends_on_row_and_tag_not_on_data():
    a = model.block_order(0, 0, 0, np.arange(64))
    b = model.block_order(0, 1, 0, np.arange(64))
    c = model.block_order(0, 0, 1, np.arange(64))
    assert a.tolist() != b.tolist() and a.tolist() != c.tolist()


# ---------------------------------------------------------------- model vs oracle

SMALL = {"gauss4k": 1, "dsa32k": 4, "dsa128k_bf16": 3, "vocab152k_k64": 2,
         "vocab152k_k1024": 2, "asc1m": 1, "ties1m": 1}


def _check_row(x_row, res, o_vals, o_idx, k):
    raw, _ = oracle.raw_bits(x_row)
    assert len(res.idx) == k
    assert len(set(res.idx.tolist())) == k
    assert np.all((res.idx >= 0) & (res.idx < len(raw)))
    assert np.array_equal(raw[res.idx], res.vals)
    assert np.array_equal(np.sort(oracle.keys(res.vals)), np.sort(oracle.keys(o_vals)))
    okeys = oracle.keys(raw)
    kth = int(oracle.keys(o_vals).min())
    if k == len(raw) or int((okeys > kth).sum()) + int((okeys == kth).sum()) == k:
        assert sorted(res.idx.tolist()) == sorted(o_idx.tolist())
    assert res.kth == kth


@pytest.mark.parametrize("name", list(SMALL))
def test_model_matches_oracle(name):
    w = synth.WORKLOADS[name]
    x = synth.generate(name, SMALL[name])
    o_vals, o_idx = oracle.topk(x, w.k)
    for r in range(x.shape[0]):
        res = model.row_topk(x[r], w.k, w.block, w.block2, seed=0, row=r)
        _check_row(x[r], res, o_vals[r], o_idx[r], w.k)
        st = res.stats
        # every element read exactly once, in blocks (deep-dive, Notes)
        assert np.all(res.reads == 1)
        # len(topk_candidate) <= k + B2 + B at all times; the check after every
        # block makes the strict bound k + B2 + B - 1
        assert st.max_len <= w.k + w.block + w.block2 - 1
        # T only rises, and everything is admitted before the first compaction
        assert all(a <= b for a, b in zip(st.thresholds, st.thresholds[1:]))
        assert st.all_admitted_before_first_compaction
        # W = A + kR and R*B2 <= A (analysis section)
        assert st.W == st.A + w.k * st.R
        assert st.R * w.block2 <= st.A


@pytest.mark.parametrize("split", [2, 3, 8])
def test_split_rows_match_oracle(split):
    for name in ("dsa32k", "asc1m_b1", "dsa128k_bf16"):
        w = synth.WORKLOADS[name]
        x = synth.generate(name, 1)
        o_vals, o_idx = oracle.topk(x, w.k)
        res = model.row_topk(x[0], w.k, w.block, w.block2, seed=4, row=0, split=split)
        _check_row(x[0], res, o_vals[0], o_idx[0], w.k)
        assert np.all(res.reads == 1)
        assert res.stats.W == res.stats.A + w.k * res.stats.R


def test_edge_shapes_match_oracle():
    cases = [
        (1, 1, 1, 1), (5, 5, 2, 1), (37, 3, 4, 5), (100, 100, 7, 3), (1000, 1, 1, 1),
        (1000, 17, 1000, 1000), (1001, 64, 256, 3), (4096, 64, 5000, 1),
    ]
    for n, k, b, b2 in cases:
        for kind in ("gauss", "small_ints", "special"):
            for dt in ("f32", "bf16"):
                x = synth.random_rows(1, n, dt, n + k, kind)
                o_vals, o_idx = oracle.topk(x, k)
                res = model.row_topk(x[0], k, b, b2, seed=1)
                _check_row(x[0], res, o_vals[0], o_idx[0], k)
                assert res.stats.max_len <= k + b + b2 - 1


def test_all_minus_inf_row_fills_the_buffer():
    x = np.full((1, 3000), 0xFF80, dtype=np.uint16)
    x[0, 17] = 0x3F80  # one finite value
    o_vals, o_idx = oracle.topk(x, 100)
    res = model.row_topk(x[0], 100, 256, 256)
    _check_row(x[0], res, o_vals[0], o_idx[0], 100)
    assert 17 in res.idx.tolist()


# ---------------------------------------------------------------- analysis

@pytest.mark.parametrize("name", ["gauss4k", "dsa32k", "dsa128k_bf16", "vocab152k_k64",
                                  "vocab152k_k1024", "asc1m", "ties1m"])
def test_mean_w_below_bound(name):
    """E[W] <= (1 + k/B2)(k+B+B2)H_m over the random block order."""
    w = synth.WORKLOADS[name]
    rows = {"gauss4k": 1, "asc1m": 1, "ties1m": 1}.get(name, 2)
    x = synth.generate(name, rows)
    seeds = range(8) if w.n <= 200000 else range(3)
    ws = [model.row_topk(x[r], w.k, w.block, w.block2, seed=s, row=r).stats.W
          for r in range(rows) for s in seeds]
    bound = model.expected_w_bound(w.n, w.k, w.block, w.block2)
    assert np.mean(ws) <= bound
    assert max(ws) <= 1.5 * bound


def test_block_order_changes_cost_not_result():
    w = synth.WORKLOADS["dsa32k"]
    x = synth.generate("dsa32k", 1)[0]
    ref = None
    for seed in range(10):
        res = model.row_topk(x, w.k, w.block, w.block2, seed=seed)
        got = sorted(res.vals.view(np.float32).tolist())
        ref = ref or got
        assert got == ref
    # in-order scan (the identity order) of an ascending row: same answer,
    # far more work than the random order
    asc = synth.generate("asc1m", 1)[0][: 1 << 17]
    keys = oracle.keys(asc)
    blocks = [(keys[lo:lo + 1024], np.arange(lo, lo + 1024)) for lo in range(0, len(asc), 1024)]
    ck, ci, kth, st = model.deepselect(blocks, 512, 1024, 32)
    assert sorted(ci.tolist()) == list(range(len(asc) - 512, len(asc)))
    rnd = model.row_topk(asc, 512, 1024, 1024, seed=0)
    assert st.W > 10 * rnd.stats.W


# ---------------------------------------------------------------- per-row valid lengths

def _prefix_check(x_row, length, k, res):
    """The model on a prefix against the oracle's plain top-k of that prefix."""
    n_valid = min(max(int(length), 0), len(x_row))
    c = min(k, n_valid)
    assert len(res.idx) == c
    if c == 0:
        return
    sub = np.ascontiguousarray(x_row[:n_valid])[None, :]
    o_vals, _ = oracle.topk(sub, c)
    assert np.all(res.idx < n_valid) and len(np.unique(res.idx)) == c
    assert np.array_equal(np.sort(oracle.keys(res.vals)), np.sort(oracle.keys(o_vals[0])))


@pytest.mark.parametrize("split", [1, 3])
def test_valid_length_prefix_matches_oracle(split):
    # the method on x[:L] for lengths across the edge cases: none, one
    # element, fewer than k, a ragged last block, fewer blocks than parts,
    # all of N, past N (clamped) and negative (clamped to 0)
    n, k, B, B2 = 5000, 96, 256, 128
    x = synth.random_rows(1, n, "f32", 5, "gauss")[0]
    for L in [0, 1, 7, k - 1, k, k + 1, 255, 257, 600, 2 * 256 + 3, n, n + 50, -4]:
        res = model.row_topk(x, k, B, B2, seed=2, row=0, split=split, length=L)
        _prefix_check(x, L, k, res)
        st = res.stats
        assert st.W == st.A + k * st.R  # per call, so also summed over parts and merge
        assert st.A <= max(0, min(L, n)) + (split > 1) * split * k
        if min(max(L, 0), n) == 0:
            assert (st.W, st.A, st.R, st.max_len) == (0, 0, 0, 0)


def test_valid_length_n_is_the_plain_row():
    w = synth.WORKLOADS["dsa32k"]
    x = synth.generate("dsa32k", 2)
    for split in (1, 2):
        a = model.row_topk(x[1], w.k, w.block, w.block2, seed=4, row=1, split=split)
        b = model.row_topk(x[1], w.k, w.block, w.block2, seed=4, row=1, split=split, length=w.n)
        assert np.array_equal(a.idx, b.idx)
        assert (a.stats.W, a.stats.A, a.stats.R, a.stats.max_len) == \
            (b.stats.W, b.stats.A, b.stats.R, b.stats.max_len)


def test_causal_lengths_mark_the_minus_inf_tail():
    # the lengths the causal workload is drawn with: finite values before,
    # -inf from there on, so the prefix holds every finite value of the row
    x = synth.generate("dsa128k_bf16", 5)
    L = synth.valid_lengths("dsa128k_bf16", range(5))
    for r in range(5):
        assert np.all(x[r, L[r]:] == 0xFF80)
        assert x[r, L[r] - 1] != 0xFF80
        assert 2048 <= L[r] <= x.shape[1]
    w = synth.WORKLOADS["dsa128k_bf16"]
    for r in range(2):
        res = model.row_topk(x[r], w.k, w.block, w.block2, seed=0, row=r, split=2, length=L[r])
        _prefix_check(x[r], L[r], w.k, res)


# ------------------------------------------------------- the bound itself

# (N, k, B, B2): the small and the long-context workloads, the logits shape
# (ceil(N/B) = 149, floor 148), a ragged case whose ceil and floor of N/B
# differ with k != B2 and B != B2, and one-block rows.
_BOUND_CASES = [(4096, 64, 256, 256), (131072, 2048, 2048, 2048), (151936, 64, 1024, 1024),
                (4097, 64, 256, 512), (1048576, 512, 1024, 1024), (100, 5, 200, 7), (200, 30, 200, 1)]
_EULER_GAMMA = 0.57721566490153286060651209


def _harmonic_asymptotic(m: int) -> float:
    """H_m by the Euler-Maclaurin series ln m + gamma + 1/2m - 1/12m^2 + 1/120m^4
    (error below 1/(252 m^6)), independent of any summation of 1/i."""
    return math.log(m) + _EULER_GAMMA + 1 / (2 * m) - 1 / (12 * m * m) + 1 / (120 * m ** 4)


def test_w_bound_one_block_is_the_leading_factor():
    """m = ceil(N/B) = 1 gives H_1 = 1: the bound is exactly (1 + k/B2)(k + B + B2)."""
    for n, k, b, b2 in [(100, 5, 200, 7), (200, 30, 200, 1), (64, 64, 64, 64)]:
        assert model.expected_w_bound(n, k, b, b2) == pytest.approx((1 + k / b2) * (k + b + b2), rel=1e-15)


def test_w_bound_known_harmonic_value():
    """H_16 = 2436559/720720 (the exact rational), so the 4096-element row with
    k = 64, B = B2 = 256 has bound 1.25 * 576 * H_16."""
    h16 = Fraction(2436559, 720720)
    assert sum(Fraction(1, i) for i in range(1, 17)) == h16  # the fraction itself
    assert model.expected_w_bound(4096, 64, 256, 256) == pytest.approx(float(Fraction(5, 4) * 576 * h16),
                                                                       rel=1e-14)


@pytest.mark.parametrize("case", [c for c in _BOUND_CASES if -(-c[0] // c[2]) >= 16])
def test_w_bound_matches_the_asymptotic_form(case):
    """The boxed bound reads (1 + k/B2) L (ln m + O(1)); the O(1) is Euler's gamma
    plus the series tail. Pins m = ceil(N/B), the factor (1 + k/B2) and L = k+B+B2."""
    n, k, b, b2 = case
    m = -(-n // b)
    lead = (1 + k / b2) * (k + b + b2)
    assert model.expected_w_bound(n, k, b, b2) / lead == pytest.approx(_harmonic_asymptotic(m), abs=1e-8)


def test_w_bound_pins_reject_plausible_mistakes():
    """Each plausible slip in the formula moves at least one pinned case."""
    def exact(n, k, b, b2):
        m = -(-n // b)
        return float((1 + Fraction(k, b2)) * (k + b + b2) * sum(Fraction(1, i) for i in range(1, m + 1)))

    def harm(m):
        return math.fsum(1.0 / i for i in range(1, m + 1))

    mutants = {
        "m = floor(N/B)": lambda n, k, b, b2: (1 + k / b2) * (k + b + b2) * harm(max(1, n // b)),
        "m = N": lambda n, k, b, b2: (1 + k / b2) * (k + b + b2) * harm(n),
        "(1 + B2/k)": lambda n, k, b, b2: (1 + b2 / k) * (k + b + b2) * harm(-(-n // b)),
        "L = k + 2B": lambda n, k, b, b2: (1 + k / b2) * (k + 2 * b) * harm(-(-n // b)),
        "no (1 + k/B2)": lambda n, k, b, b2: (k + b + b2) * harm(-(-n // b)),
    }
    for name, f in mutants.items():
        assert any(abs(f(*c) - exact(*c)) > 1e-6 * exact(*c) for c in _BOUND_CASES), name
    for c in _BOUND_CASES:
        assert model.expected_w_bound(*c) == pytest.approx(exact(*c), rel=1e-13), c


def test_w_bound_of_split_rows():
    """Split rows (reading c12): the parts' bounds with their own m_s plus the
    merge's, a DeepSelect over S blocks of k. Worked by hand for a 4096-element
    row, k = 64, B = B2 = 256, S = 2: two parts of 8 blocks (H_8 = 761/280)
    and a merge of two blocks of 64 (H_2 = 3/2, L = 64 + 64 + 256)."""
    want = 2 * Fraction(5, 4) * 576 * Fraction(761, 280) + Fraction(5, 4) * 384 * Fraction(3, 2)
    assert model.expected_w_bound_row(4096, 64, 256, 256, 2) == pytest.approx(float(want), rel=1e-13)
    assert model.expected_w_bound_row(4096, 64, 256, 256, 1) == model.expected_w_bound(4096, 64, 256, 256)
    # uneven parts: 17 blocks (the last holds 1 element) over 3 parts of 5, 6 and 6 blocks
    n, k, b, b2 = 4097, 16, 256, 128
    parts = [(0, 5), (5, 11), (11, 17)]
    assert model.part_bounds(17, 3) == parts
    hm = lambda m: sum(Fraction(1, i) for i in range(1, m + 1))
    lead = (1 + Fraction(k, b2)) * (k + b + b2)
    want = lead * (hm(5) + hm(6) + hm(6)) + (1 + Fraction(k, b2)) * (k + k + b2) * hm(3)
    assert model.expected_w_bound_row(n, k, b, b2, 3) == pytest.approx(float(want), rel=1e-13)


def test_split_rows_mean_w_below_their_bound():
    """The model's W of split rows (parts plus merge) stays under the summed bound."""
    for name, split in [("dsa32k", 4), ("dsa128k_bf16", 2), ("asc1m", 8)]:
        w = synth.WORKLOADS[name]
        x = synth.generate(name, 1)
        ws = [model.row_topk(x[0], w.k, w.block, w.block2, seed=s, split=split).stats.W for s in range(3)]
        assert np.mean(ws) <= model.expected_w_bound_row(w.n, w.k, w.block, w.block2, split), name


def test_merge_starts_below_the_largest_part_kth():
    """Reading c12: the merge admits only part results at or above the largest
    k-th key among the parts (no part's k-th exceeds the row's k-th)."""
    k, b, b2 = 16, 64, 32
    # ascending row in 4 parts: the top part holds the row's top k, every other
    # result lies below its k-th, so the merge admits exactly k results and
    # only runs its final select (W = k, A = k, R = 0)
    x = np.arange(1024, dtype=np.float32)[None, :]
    full = model.row_topk(x[0], k, b, b2, seed=3, split=4)
    keys = oracle.keys(x[0])
    parts = 0
    for lo, hi in model.part_bounds(16, 4):  # each part on its own blocks, in the row's order
        blocks = [(keys[i * b:(i + 1) * b], np.arange(i * b, (i + 1) * b))
                  for i in model.block_order(3, 0, 0, np.arange(lo, hi))]
        parts += model.deepselect(blocks, k, b2, 32)[3].W
    o_vals, o_idx = oracle.topk(x, k)
    assert sorted(full.idx.tolist()) == sorted(o_idx[0].tolist())
    assert full.stats.W - parts == k
    # the merge on its own: blocks of part results with t0 = the largest k-th
    blocks = [(np.arange(100, 116, dtype=np.uint32), np.arange(16)),
              (np.arange(300, 316, dtype=np.uint32), np.arange(16, 32)),
              (np.arange(200, 216, dtype=np.uint32), np.arange(32, 48))]
    ck, ci, kth, st = model.deepselect(blocks, k, b2, 32, t0=300)
    assert st.A == 16 and st.R == 0 and st.W == 16 and kth == 300
    assert sorted(ck.tolist()) == list(range(300, 316))
    # ties at t0 are admitted (>=): every result equal
    eq = [(np.full(16, 7, dtype=np.uint32), np.arange(16 * i, 16 * i + 16)) for i in range(3)]
    ck, ci, kth, st = model.deepselect(eq, k, b2, 32, t0=7)
    assert st.A == 48 and kth == 7 and len(ck) == k
    assert st.W == st.A + k * st.R
