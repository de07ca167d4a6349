"""Fused sampling over a row's top-k results -- TEST INFRASTRUCTURE ONLY.

The definitions the GPU's fused sampling is checked against, in float64:

* the softmax of the k selected values at a temperature: each value's
  exponential, taken after subtracting the largest value, over their sum (the
  max-subtracted softmax of "常见CUDA手写实现", section on softmax);
* nucleus (top-p) truncation: the smallest prefix of the results, largest
  first, whose probability reaches p;
* one draw by the inverse of the cumulative distribution over that prefix in
  the same order: the first position whose running probability exceeds u
  times the prefix's probability.

A row whose largest value is +inf takes the limit of the softmax as that
value grows without bound: the +inf results share the mass equally and every
other result gets 0 (the max-subtracted form would give inf - inf).

The top-k step itself is the sampling use the DeepSelect deep-dive names in
its section "算法设计背景" (top-k over vocabulary logits).
"""
from __future__ import annotations

import numpy as np

from oracle import raw_bits

F32_NEG_INF_BITS = 0xFF800000


def values_of(raw_row: np.ndarray) -> np.ndarray:
    """float64 values of raw float32 (uint32) or bfloat16 (uint16) patterns."""
    raw, dt = raw_bits(np.asarray(raw_row))
    bits = raw.astype(np.uint32) if dt == 0 else raw.astype(np.uint32) << np.uint32(16)
    return bits.view(np.float32).astype(np.float64)


def softmax(values_desc: np.ndarray, temperature: float = 1.0) -> np.ndarray:
    """Probabilities of values given largest first (float64). A row whose
    largest value is not above -inf (or is NaN, or is empty) gets all zeros;
    -inf and NaN values get probability 0; when the largest value is +inf the
    +inf values share the mass equally (the limit of the softmax)."""
    v = np.asarray(values_desc, dtype=np.float64)
    if len(v) == 0 or not (v[0] > -np.inf) or np.isnan(v[0]):
        return np.zeros(len(v))
    if v[0] == np.inf:
        e = (v == np.inf).astype(np.float64)
        return e / e.sum()
    fin = v > -np.inf  # False for -inf and NaN
    e = np.where(fin, np.exp(np.where(fin, v - v[0], 0.0) / temperature), 0.0)
    return e / e.sum()


def nucleus_end(probs: np.ndarray, top_p: float) -> int:
    """Last position of the smallest prefix whose probability reaches top_p."""
    c = np.cumsum(probs)
    hit = np.nonzero(c >= top_p)[0]
    return int(hit[0]) if len(hit) else len(probs) - 1


def sample_position(probs: np.ndarray, top_p: float, u: float) -> int:
    """Inverse-CDF draw inside the nucleus: the first position whose running
    probability exceeds u times the nucleus probability (-1 for an empty or
    all-zero row)."""
    if len(probs) == 0 or probs.sum() == 0.0:
        return -1
    jp = nucleus_end(probs, top_p)
    c = np.cumsum(probs[:jp + 1])
    hit = np.nonzero(c > u * c[-1])[0]
    return int(hit[0]) if len(hit) else jp


__all__ = ["values_of", "softmax", "nucleus_end", "sample_position"]
