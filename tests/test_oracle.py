"""Pins of the CPU oracle (``oracle/``) against things other than itself.

Each test fixes the oracle with a fact the pages or the mathematics state:
the pages' worked example, brute force over tiny rows with an independently
written value order, closed forms of the structured workloads, and numpy's
own sort of the values.
"""
import itertools
import json
import math
import os
import struct

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


def bits_f32(u: int) -> float:
    return struct.unpack("<f", struct.pack("<I", u & 0xFFFFFFFF))[0]


def independent_order(u: int, width: int):
    """Sort key of a raw pattern written from float semantics, not from bit tricks.

    negative NaN < -inf < ... < -0 < +0 < ... < +inf < positive NaN; two NaNs
    of one sign compare by payload magnitude (larger payload further out).
    """
    v = bits_f32(u if width == 32 else u << 16)
    sign = (u >> (width - 1)) & 1
    if math.isnan(v):
        payload = u & ((1 << (width - 1)) - 1)
        return (0, -payload) if sign else (2, payload)
    zero_rank = 0 if (v == 0.0 and sign) else 1
    return (1, v, zero_rank)


# ---------------------------------------------------------------- worked example

def test_worked_example_from_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "topk_worked_example.json")))
    x = np.array([g["input"]], dtype=np.float32)
    vals, idx = oracle.topk(x, g["k"])
    assert vals.view(np.float32)[0].tolist() == g["output_descending"]
    assert sorted(idx[0].tolist()) == [1, 2, 4]


# ---------------------------------------------------------------- brute force

ALPHABET32 = [f32_bits(v) for v in (-math.inf, -1.0, -0.0, 0.0, 1.0, math.inf)] + [
    0x7FC00000, 0xFFC00000]


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_brute_force_all_tiny_rows_f32(n):
    rows = np.array(list(itertools.product(ALPHABET32, repeat=n)), dtype=np.uint32)
    for k in range(1, n + 1):
        vals, idx = oracle.topk(rows, k)
        for r in range(rows.shape[0]):
            row = rows[r].tolist()
            chosen = idx[r].tolist()
            assert len(set(chosen)) == k and all(0 <= i < n for i in chosen)
            assert vals[r].tolist() == [row[i] for i in chosen]
            order = [independent_order(u, 32) for u in row]
            rest = [i for i in range(n) if i not in chosen]
            if rest:
                # every kept element is >= every dropped one ...
                assert min(order[i] for i in chosen) >= max(order[i] for i in rest)
                # ... and among equal values the lowest indices are kept
                kth = min(order[i] for i in chosen)
                ties_kept = sorted(i for i in chosen if order[i] == kth)
                ties_all = sorted(i for i in range(n) if order[i] == kth)
                assert ties_kept == ties_all[:len(ties_kept)]
            # output is in descending value order
            assert [order[i] for i in chosen] == sorted((order[i] for i in chosen), reverse=True)


def test_brute_force_random_tiny_rows_bf16():
    rng = np.random.default_rng(11)
    alphabet = np.array([0xFF80, 0xBF80, 0x8000, 0x0000, 0x3F80, 0x7F80, 0x7FC0, 0xFFC0,
                         0x0001, 0x8001], dtype=np.uint16)
    rows = alphabet[rng.integers(0, len(alphabet), (3000, 6))]
    for k in (1, 3, 6):
        vals, idx = oracle.topk(rows, k)
        for r in range(rows.shape[0]):
            row = rows[r].tolist()
            order = [independent_order(u, 16) for u in row]
            # stable sort by descending value: equal values keep index order
            by_desc = sorted(range(6), key=lambda i: tuple(-c for c in order[i]))
            assert idx[r].tolist() == by_desc[:k]
            assert vals[r].tolist() == [row[i] for i in by_desc[:k]]


# ---------------------------------------------------------------- key transform

def test_key16_is_a_bijection_and_follows_float_order():
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    k = oracle.keys(pats)
    assert sorted(k.tolist()) == list(range(1 << 16))
    ordered = sorted(range(1 << 16), key=lambda u: independent_order(u, 16))
    assert [int(k[u]) for u in ordered] == list(range(1 << 16))


def test_key32_edges_and_random_pairs_follow_float_order():
    edges = [0x00000000, 0x80000000, 0x00000001, 0x80000001, 0x007FFFFF, 0x807FFFFF,
             0x00800000, 0x80800000, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F800000, 0xFF800000,
             0x7FC00000, 0xFFC00000, 0x7F800001, 0xFF800001, 0x7FFFFFFF, 0xFFFFFFFF,
             0x3F800000, 0xBF800000]
    rng = np.random.default_rng(5)
    sample = np.concatenate([np.array(edges, dtype=np.uint32),
                             rng.integers(0, 1 << 32, 200000, dtype=np.uint64).astype(np.uint32)])
    k = oracle.keys(sample)
    for _ in range(3):
        a = rng.integers(0, len(sample), 100000)
        b = rng.integers(0, len(sample), 100000)
        for i, j in zip(a[:20000], b[:20000]):
            oi = independent_order(int(sample[i]), 32)
            oj = independent_order(int(sample[j]), 32)
            assert (k[i] < k[j]) == (oi < oj)
            assert (k[i] == k[j]) == (sample[i] == sample[j])


def test_c_key_matches_python_key():
    pats = np.arange(1 << 16, dtype=np.uint32)
    py = oracle.keys(pats.astype(np.uint16))
    assert all(oracle.key_c(oracle.BF16, int(u)) == int(py[u]) for u in range(0, 1 << 16, 7))
    rng = np.random.default_rng(3)
    s = rng.integers(0, 1 << 32, 5000, dtype=np.uint64).astype(np.uint32)
    py32 = oracle.keys(s)
    assert all(oracle.key_c(oracle.F32, int(u)) == int(v) for u, v in zip(s, py32))


# ---------------------------------------------------------------- closed forms

def test_ascending_rows_closed_form():
    x = synth.generate("asc1m", 2)
    k = 512
    vals, idx = oracle.topk(x, k)
    n = x.shape[1]
    for r in range(2):
        assert idx[r].tolist() == list(range(n - 1, n - 1 - k, -1))
        assert vals[r].view(np.float32).tolist() == [float(i) for i in range(n - 1, n - 1 - k, -1)]


def test_heavy_ties_closed_form():
    x = synth.generate("ties1m", 2)
    k = 512
    vals, idx = oracle.topk(x, k)
    for r in range(2):
        top = np.flatnonzero(x[r] == np.float32(7.5))
        assert len(top) > 50000  # about N/16
        assert np.all(vals[r].view(np.float32) == np.float32(7.5))
        assert idx[r].tolist() == top[:k].tolist()


def test_values_match_numpy_sort():
    for name, rows in (("dsa32k", 3), ("dsa128k_bf16", 3), ("vocab152k_k64", 2)):
        w = synth.WORKLOADS[name]
        x = synth.generate(name, rows)
        vals, idx = oracle.topk(x, w.k)
        xf = x if w.dtype == "f32" else synth.bf16_bits_to_f32(x)
        for r in range(rows):
            expect = np.sort(xf[r])[::-1][:w.k]
            got = vals[r].view(np.float32) if w.dtype == "f32" else synth.bf16_bits_to_f32(vals[r])
            assert np.array_equal(got, expect)
            assert np.array_equal(xf[r][idx[r]], got)


def test_k_equals_n_and_k_one():
    x = synth.random_rows(3, 37, "f32", 9, "small_ints")
    vals, idx = oracle.topk(x, 37)
    assert all(sorted(idx[r].tolist()) == list(range(37)) for r in range(3))
    vals, idx = oracle.topk(x, 1)
    for r in range(3):
        assert idx[r, 0] == int(np.flatnonzero(x[r] == x[r].max())[0])


def test_oracle_rejects_bad_arguments():
    x = np.zeros((2, 8), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.topk(x, 0)
    with pytest.raises(ValueError):
        oracle.topk(x, 9)
