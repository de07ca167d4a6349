"""Seeded synthetic rows for batched row-wise top-k.

This module only makes inputs. It holds none of the selection arithmetic and is
shared by the CPU oracle side (``oracle/``, ``tests/``) and the benchmark.

The workloads stand in for the two uses that the DeepSelect deep-dive
(PFCCLab/DeepSelect, "算法设计背景") names: top-k over DeepSeek Sparse
Attention indexer scores across many context tokens, and top-k over a large
sampling vocabulary. Real indexer scores or logits would need trained weights,
so every row is synthetic:

* ``gauss4k``        1 x 4096 float32, iid N(0,1);            k=64,   B=B2=256
* ``dsa32k``         64 x 32768 float32, iid N(0,1);          k=512,  B=B2=1024
* ``dsa128k_bf16``   128 x 131072 bfloat16, iid N(0,1) with a causal valid
                     length L_r ~ UniformInt[2048, 131072] and -inf from L_r on;
                                                             k=2048, B=B2=2048
* ``vocab152k_k64``  256 x 151936 float32 logits
                     -1.1*ln(rank+1) + 0.5*z, rank a per-row random permutation
                     of 0..N-1, z ~ N(0,1) (computed in float64, cast to
                     float32);                                k=64,   B=B2=1024
* ``vocab152k_k1024`` same rows;                              k=1024, B=B2=1024
* ``asc1m``          32 x 1048576 float32, x[r, i] = i (strictly ascending,
                     the worst case for scanning in order);    k=512,  B=B2=1024
* ``ties1m``         32 x 1048576 float32, uniform over the 16 values
                     -7.5, -6.5, ..., 7.5 (heavy ties);        k=512,  B=B2=1024
* ``asc1m_b1``       1 x 1048576 ascending (one row: the split-row path)

Each row r of a workload is drawn from its own PCG64 stream seeded with
``(data_seed, r)``, so a row does not depend on how many rows are generated
and any single row of a full-size batch can be regenerated alone.

float32 rows are returned as ``numpy.float32``; bfloat16 rows as ``numpy.uint16``
holding the raw bfloat16 bit patterns (round-to-nearest-even of the float32
draw, done in integer arithmetic).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

BF16_NEG_INF = np.uint16(0xFF80)


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n: int
    dtype: str  # "f32" or "bf16"
    k: int
    block: int  # B
    block2: int  # B2
    data_seed: int
    kind: str  # generator family
    about: str

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS = {
    w.name: w
    for w in [
        Workload("gauss4k", 1, 4096, "f32", 64, 256, 256, 1, "gauss",
                 "one row of 4096 iid N(0,1) float32 scores"),
        Workload("dsa32k", 64, 32768, "f32", 512, 1024, 1024, 2, "gauss",
                 "64 indexer-score rows of 32768 iid N(0,1) float32"),
        Workload("dsa128k_bf16", 128, 131072, "bf16", 2048, 2048, 2048, 3, "causal",
                 "128 long-context bf16 score rows, random causal length, -inf tail"),
        Workload("vocab152k_k64", 256, 151936, "f32", 64, 1024, 1024, 4, "logits",
                 "256 vocabulary logit rows (Zipf-like rank decay plus noise), k=64"),
        Workload("vocab152k_k1024", 256, 151936, "f32", 1024, 1024, 1024, 4, "logits",
                 "256 vocabulary logit rows (Zipf-like rank decay plus noise), k=1024"),
        Workload("asc1m", 32, 1 << 20, "f32", 512, 1024, 1024, 5, "ascending",
                 "32 strictly ascending rows of 2^20 float32"),
        Workload("ties1m", 32, 1 << 20, "f32", 512, 1024, 1024, 55, "ties16",
                 "32 rows of 2^20 float32 drawn from 16 distinct values"),
        Workload("asc1m_b1", 1, 1 << 20, "f32", 512, 1024, 1024, 5, "ascending",
                 "one strictly ascending row of 2^20 float32"),
    ]
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return raw uint16 bits.

    Inputs must be finite or infinite (no NaN); the synthetic rows never hold NaN.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 bits to float32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _row(w: Workload, r: int) -> np.ndarray:
    rng = np.random.default_rng((w.data_seed, r))
    n = w.n
    if w.kind == "gauss":
        return rng.standard_normal(n, dtype=np.float32)
    if w.kind == "causal":
        vals = f32_to_bf16_bits(rng.standard_normal(n, dtype=np.float32))
        valid = int(rng.integers(2048, n, endpoint=True))
        vals[valid:] = BF16_NEG_INF
        return vals
    if w.kind == "logits":
        rank = rng.permutation(n).astype(np.float64)
        z = rng.standard_normal(n)
        return (-1.1 * np.log(rank + 1.0) + 0.5 * z).astype(np.float32)
    if w.kind == "ascending":
        return np.arange(n, dtype=np.float32)
    if w.kind == "ties16":
        return (rng.integers(0, 16, n).astype(np.float32) - np.float32(7.5)).astype(np.float32)
    raise ValueError(f"unknown generator family {w.kind!r}")


def valid_lengths(name: str, rows=None) -> np.ndarray:
    """Per-row valid length (int32) of workload ``name``: where a causal row's
    -inf tail starts, N for every other family. The same draws as the rows."""
    w = WORKLOADS[name]
    rows = list(range(w.batch) if rows is None else rows)
    out = np.full(len(rows), w.n, dtype=np.int32)
    if w.kind == "causal":
        for i, r in enumerate(rows):
            rng = np.random.default_rng((w.data_seed, r))
            rng.standard_normal(w.n, dtype=np.float32)
            out[i] = int(rng.integers(2048, w.n, endpoint=True))
    return out


def generate_rows(name: str, rows=None) -> np.ndarray:
    """Rows of workload ``name`` as a [len(rows), N] array (all rows if None)."""
    w = WORKLOADS[name]
    if rows is None:
        rows = range(w.batch)
    rows = list(rows)
    dt = np.float32 if w.dtype == "f32" else np.uint16
    out = np.empty((len(rows), w.n), dtype=dt)
    for i, r in enumerate(rows):
        if not 0 <= r < w.batch:
            raise IndexError(f"row {r} outside workload {name} (batch {w.batch})")
        out[i] = _row(w, r)
    return out


def generate(name: str, batch=None) -> np.ndarray:
    """The first ``batch`` rows of workload ``name`` (the full batch if None)."""
    w = WORKLOADS[name]
    return generate_rows(name, range(w.batch if batch is None else batch))


def random_rows(batch: int, n: int, dtype: str, seed: int, kind: str = "gauss") -> np.ndarray:
    """Ad-hoc seeded rows for edge-case tests (shape and distribution chosen by caller).

    kinds: ``gauss`` N(0,1); ``small_ints`` integers in [-3, 3] (many ties);
    ``special`` a mix of +-0, +-inf, denormals and ordinary values.
    """
    rng = np.random.default_rng((seed, batch, n))
    if kind == "gauss":
        x = rng.standard_normal((batch, n), dtype=np.float32)
    elif kind == "small_ints":
        x = rng.integers(-3, 4, (batch, n)).astype(np.float32)
    elif kind == "special":
        pool = np.array([0.0, -0.0, np.inf, -np.inf, 1e-40, -1e-40, 1.0, -1.0, 3.5,
                         -2.25, 65504.0, -1e30], dtype=np.float32)
        x = pool[rng.integers(0, len(pool), (batch, n))]
    else:
        raise ValueError(kind)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    return f32_to_bf16_bits(x).reshape(batch, n)
