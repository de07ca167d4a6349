"""The seeded input generators: bf16 rounding and the workloads' stated structure."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, np.inf, -np.inf, 1e-40, -3.0e38], dtype=np.float32),
                        rng.integers(0, 1 << 31, 50000).astype(np.uint32).view(np.float32)])
    x = x[np.isfinite(x) | np.isinf(x)]
    x = x[~np.isnan(x)]
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(synth.bf16_bits_to_f32(ours),
                          torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_rows_are_independent_of_batch_size():
    a = synth.generate("dsa32k", 3)
    b = synth.generate_rows("dsa32k", [2])
    assert np.array_equal(a[2], b[0])


def test_causal_rows_have_a_minus_inf_tail():
    x = synth.generate("dsa128k_bf16", 8)
    for r in range(8):
        finite = np.flatnonzero(x[r] != synth.BF16_NEG_INF)
        valid = finite.max() + 1
        assert 2048 <= valid <= 131072
        assert np.all(x[r, valid:] == synth.BF16_NEG_INF)


def test_logit_rows_decay_with_rank():
    x = synth.generate("vocab152k_k64", 1)[0]
    assert x.dtype == np.float32 and len(x) == 151936
    assert x.max() < 3.0 and x.min() < -11.0


def test_structured_rows():
    a = synth.generate("asc1m", 1)[0]
    assert np.array_equal(a, np.arange(1 << 20, dtype=np.float32))
    t = synth.generate("ties1m", 1)[0]
    assert sorted(set(t.tolist())) == [v - 7.5 for v in range(16)]
