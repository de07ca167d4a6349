"""The allocation-free entry point (deepselect_topk_noalloc) against
deepselect_topk_ex on the same inputs, through the C ABI.

Both run the same kernels with the same split, so results, tie choices and
statistics must be identical; the results are also checked against the oracle.
Two calls in a row (the second smaller) reuse the GPU's static scratch; a call
whose split workspace exceeds the scratch is refused before anything is queued.
"""
import sys

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU", allow_module_level=True)

import top_selection_row_amd as ds  # noqa: E402

DEV = torch.device("cuda:0")


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(x):
    if x.dtype == np.float32:
        return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)


def raw_of(t):
    if t.dtype == torch.float32:
        return t.cpu().numpy().view(np.uint32)
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run(entry, xt, k, B, B2, seed, split, share=0, srt=0):
    batch, n = xt.shape
    dt = ds.DS_F32 if xt.dtype == torch.float32 else ds.DS_BF16
    vals = torch.empty((batch, k), dtype=xt.dtype, device=DEV)
    idx = torch.empty((batch, k), dtype=torch.int32, device=DEV)
    st = torch.empty((batch, 4), dtype=torch.int64, device=DEV)
    stream = torch.cuda.current_stream(DEV).cuda_stream
    rc = entry(xt.data_ptr(), dt, batch, n, n, k, B, B2, seed, vals.data_ptr(), idx.data_ptr(), stream,
               split=split, stats=st.data_ptr(), sorted=srt, share_threshold=share)
    assert rc == ds.DS_OK, ds.deepselect_status_string(rc)
    torch.cuda.synchronize()
    return raw_of(vals), idx.cpu().numpy(), st.cpu().numpy()


def check_oracle(x, vals, idx, k):
    raw, _ = oracle.raw_bits(x)
    o_vals, _ = oracle.topk(x, k)
    for r in range(x.shape[0]):
        assert len(np.unique(idx[r])) == k
        assert np.array_equal(raw[r][idx[r]], vals[r])
        assert np.array_equal(np.sort(oracle.keys(vals[r])), np.sort(oracle.keys(o_vals[r])))


CASES = [
    # (workload, rows, split, sorted, shared thresholds); the second of each
    # pair is smaller than the first
    ("dsa128k_bf16", 24, 2, 0, 0),
    ("dsa32k", 4, 4, 0, 0),
    ("asc1m_b1", 1, 16, 1, 1),
    ("gauss4k", 1, 2, 0, 0),
]


def test_noalloc_matches_the_allocating_call_twice():
    for name, rows, split, srt, share in CASES:
        w = synth.WORKLOADS[name]
        log(f"[gpu] no-alloc entry {name} rows {rows} split {split} sorted {srt} share {share}")
        x = synth.generate(name, rows)
        xt = to_device(x)
        need = ds.deepselect_workspace_bytes(ds.DS_F32 if w.dtype == "f32" else ds.DS_BF16, rows, w.n, w.k,
                                             w.block, w.block2, split)
        assert 0 < need <= ds.deepselect_scratch_bytes()
        ref = run(ds.deepselect_topk_ex, xt, w.k, w.block, w.block2, 7, split, share, srt)
        got = run(ds.deepselect_topk_noalloc, xt, w.k, w.block, w.block2, 7, split, share, srt)
        check_oracle(x, got[0], got[1], w.k)
        if share:
            # thresholds shared between parts make the cost timing-dependent;
            # the result set is fixed
            for r in range(rows):
                assert np.array_equal(np.sort(oracle.keys(got[0][r])), np.sort(oracle.keys(ref[0][r])))
            assert np.all(got[2][:, 0] == got[2][:, 1] + w.k * got[2][:, 2])
        else:
            assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
            assert np.array_equal(got[2], ref[2])


def test_noalloc_shared_cells_left_zero():
    # the scratch's reserved threshold cells stay zero from call to call: a
    # call on much smaller values right after one on larger values (batches
    # below and above the 1024 reserved cells) gets the same result set as the
    # allocating call
    rng = np.random.default_rng(32)
    n, k, B, S = 65536, 16, 512, 2  # 8 or 16 ring steps per wave: the parts share thresholds
    for rows, shift in [(3, 1000.0), (5, 0.0), (1100, 2000.0), (1100, -10.0), (2, -3000.0)]:
        log(f"[gpu] no-alloc shared cells: rows {rows} shift {shift}")
        x = (rng.random((rows, n), dtype=np.float32) * np.float32(100.0) + np.float32(shift)).astype(np.float32)
        xt = to_device(x)
        ref = run(ds.deepselect_topk_ex, xt, k, B, B, 5, S, 1)
        got = run(ds.deepselect_topk_noalloc, xt, k, B, B, 5, S, 1)
        top = -np.sort(np.partition(-x, k - 1, axis=1)[:, :k], axis=1)
        for vals, idx, st in (ref, got):
            v = vals.view(np.float32)
            assert np.array_equal(-np.sort(-v, axis=1), top)
            assert np.array_equal(np.take_along_axis(x, idx.astype(np.int64), axis=1), v)
            assert np.all(st[:, 0] == st[:, 1] + k * st[:, 2])


def test_noalloc_refuses_a_workspace_beyond_the_scratch():
    # 4096 rows of 4096 bfloat16 split 4 ways at k = 512 need 64 MiB of part results
    batch, n, k, B = 4096, 4096, 512, 512
    need = ds.deepselect_workspace_bytes(ds.DS_BF16, batch, n, k, B, B, 4)
    assert need > ds.deepselect_scratch_bytes()
    xt = torch.zeros((batch, n), dtype=torch.bfloat16, device=DEV)
    vals = torch.empty((batch, k), dtype=torch.bfloat16, device=DEV)
    idx = torch.full((batch, k), -7, dtype=torch.int32, device=DEV)
    stream = torch.cuda.current_stream(DEV).cuda_stream
    rc = ds.deepselect_topk_noalloc(xt.data_ptr(), ds.DS_BF16, batch, n, n, k, B, B, 0, vals.data_ptr(),
                                    idx.data_ptr(), stream, split=4)
    torch.cuda.synchronize()
    assert rc == ds.DS_ERR_SCRATCH
    assert bool((idx == -7).all()), "a refused call wrote its output"
