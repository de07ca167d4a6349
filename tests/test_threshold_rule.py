"""The block filter's threshold test on raw bits, against the key order.

DeepSelect's block filter admits an element when it is above the threshold T
in the order of the order-preserving key transform ("改造 Radix Sort": flip
the sign bit of a positive value, every bit of a negative one). The kernels
never form that key for the test: they compare the raw bits in one integer
compare whose kind is fixed by T's sign,

  T >= +0 : key(x) > key(T)  <=>  (signed) x > (signed) t
  T <  0  : key(x) > key(T)  <=>  (unsigned) x < (unsigned) t

with bfloat16 held in the top half of a 32-bit word, whatever its low half
holds, against the padded threshold t << 16 | 0xFFFF (T >= +0) or t << 16
(T < 0); and for bfloat16 pairs also as one saturating 16-bit subtract whose
sign is the test (t - h < 0, or (h ^ 0x8000) - (t ^ 0x8000) < 0).

These rules are restated here from that description and checked against the
oracle's key transform: over every pair of 16-bit patterns (2^32 pairs, with
the low half at both extremes and at random), and for float32 over every
pair of a set of special and random patterns plus random pairs. NaN patterns
are included: the rule and the key order agree on them too.
"""
import pathlib
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ALL16 = np.arange(1 << 16, dtype=np.uint32)


def _signed32(u):
    return u.astype(np.uint32).view(np.int32).astype(np.int64)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_bf16_rule_matches_key_order_for_every_pair(tmp_path):
    """Every pair of 16-bit patterns, by tests/threshold_rule_check.c (a loop
    in C: 2^32 pairs, four forms each), against the oracle's keys."""
    table = tmp_path / "key16.bin"
    oracle.keys(ALL16.astype(np.uint16)).astype("<u4").tofile(table)
    exe = tmp_path / "threshold_rule_check"
    src = pathlib.Path(__file__).with_name("threshold_rule_check.c")
    subprocess.run(["gcc", "-std=c11", "-O3", str(src), "-o", str(exe)], check=True, timeout=300)
    res = subprocess.run([str(exe), str(table)], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 mismatches" in res.stdout


def _key32(u):
    return oracle.keys(u.astype(np.uint32).view(np.float32)).astype(np.int64)


def _rule32(x, t):
    neg = _key32(t) < 0x80000000
    unsigned = x.astype(np.int64) < t.astype(np.int64)
    signed = _signed32(x) > _signed32(t)
    return np.where(neg, unsigned, signed)


def _special32():
    s = [0x00000000, 0x80000000, 0x00000001, 0x80000001, 0x007FFFFF, 0x807FFFFF, 0x00800000,
         0x80800000, 0x3F800000, 0xBF800000, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F800000, 0xFF800000,
         0x7F800001, 0xFF800001, 0x7FC00000, 0xFFC00000, 0x7FFFFFFF, 0xFFFFFFFF, 0x3F7FFFFF,
         0xBF7FFFFF, 0x7FFFFFFE, 0xFFFFFFFE, 0x40000000, 0xC0000000]
    return np.array(s, dtype=np.uint32)


def test_f32_rule_matches_key_order_on_special_and_random_pairs():
    rng = np.random.default_rng(3)
    pats = np.concatenate([_special32(), rng.integers(0, 1 << 32, size=600, dtype=np.uint64).astype(np.uint32)])
    pats = np.concatenate([pats, pats + 1, pats - 1])  # neighbours of each
    x = np.repeat(pats, len(pats))
    t = np.tile(pats, len(pats))
    want = _key32(x) > _key32(t)
    got = _rule32(x, t)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"value {x[bad[0]]:#010x}, threshold {t[bad[0]]:#010x}"
    xr = rng.integers(0, 1 << 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    tr = rng.integers(0, 1 << 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(_rule32(xr, tr), _key32(xr) > _key32(tr))


def test_rules_reject_a_planted_mistake():
    """The bfloat16 check would catch the plausible mistakes: an unpadded
    threshold at T >= +0, or a signed compare for T < 0."""
    KEY16 = oracle.keys(ALL16.astype(np.uint16)).astype(np.int64)
    tp = ALL16[0x8000:0x8000 + 64]  # T < 0 patterns
    tp_pos = ALL16[0x3F00:0x3F40]   # T >= +0 patterns
    w = (ALL16 << 16) | 0xFFFF
    want_pos = KEY16[None, :] > KEY16[tp_pos][:, None]
    unpadded = _signed32(w)[None, :] > _signed32(tp_pos.astype(np.uint32) << 16)[:, None]
    assert np.any(unpadded != want_pos)
    want_neg = KEY16[None, :] > KEY16[tp][:, None]
    signed_for_neg = _signed32(ALL16 << 16)[None, :] > _signed32(tp.astype(np.uint32) << 16)[:, None]
    assert np.any(signed_for_neg != want_neg)
