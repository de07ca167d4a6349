"""GPU parity: the HIP DeepSelect path against the CPU oracle, through the C ABI.

Acceptance per row (bit-exact; no floating-point arithmetic happens on either
side, every comparison is an integer comparison of order-preserving keys):
  1. exactly k entries, indices distinct and in [0, N);
  2. each returned value is bit-identical to x[row, idx];
  3. the multiset of returned keys equals the oracle's;
  4. when the k-th value does not tie across the cut, the index set equals the
     oracle's (with a tie, several index sets are correct and (1)-(3) decide).
W, A, R and max_len per row must equal the method model's exactly: they do not
depend on which tied elements survive, only on the block order and the data.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from oracle import model
from oracle import sampling as oracle_sampling

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU", allow_module_level=True)

import top_selection_row_amd as ds  # noqa: E402

DEV = torch.device("cuda:0")


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(x: np.ndarray):
    if x.dtype == np.float32:
        return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)


def raw_of(t):
    if t.dtype == torch.float32:
        return t.cpu().numpy().view(np.uint32)
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    raise TypeError(t.dtype)


def run_gpu(x: np.ndarray, k, B, B2, seed=0, split=0, stats=True, waves=0, kernel=0, sorted=False):
    xt = to_device(x)
    out = ds.topk(xt, k, B, B2, seed, split=split, stats=stats, waves=waves, kernel=kernel, sorted=sorted)
    torch.cuda.synchronize()
    vals, idx = raw_of(out[0]), out[1].cpu().numpy()
    st = out[2].cpu().numpy() if stats else None
    return vals, idx, st


def check_rows(x: np.ndarray, vals, idx, k, rows=None):
    raw, _ = oracle.raw_bits(x)
    o_vals, o_idx = oracle.topk(x, k)
    rows = range(x.shape[0]) if rows is None else rows
    n = x.shape[1]
    for r in rows:
        assert idx[r].shape == (k,)
        assert len(np.unique(idx[r])) == k, f"row {r}: repeated index"
        assert idx[r].min() >= 0 and idx[r].max() < n, f"row {r}: index out of range"
        assert np.array_equal(raw[r][idx[r]], vals[r]), f"row {r}: value bits differ from x[idx]"
        got = np.sort(oracle.keys(vals[r]))
        want = np.sort(oracle.keys(o_vals[r]))
        assert np.array_equal(got, want), f"row {r}: top-k multiset differs from the oracle"
        keys_r = oracle.keys(raw[r])
        kth = want[0]
        if k == n or int((keys_r >= kth).sum()) == k:
            assert np.array_equal(np.sort(idx[r]), np.sort(o_idx[r])), f"row {r}: index set differs"


def check_sorted_rows(x: np.ndarray, vals, idx, k, rows=None):
    """Sorted output: the oracle's (key desc, column asc) order, exactly.

    Keys match the oracle position by position; equal keys come by ascending
    column; every entry above the k-th key is the oracle's own; when no tie
    crosses the cut the whole index array is the oracle's.
    """
    raw, _ = oracle.raw_bits(x)
    o_vals, o_idx = oracle.topk(x, k)
    n = x.shape[1]
    rows = range(x.shape[0]) if rows is None else rows
    for r in rows:
        assert len(np.unique(idx[r])) == k, f"row {r}: repeated index"
        assert idx[r].min() >= 0 and idx[r].max() < n, f"row {r}: index out of range"
        assert np.array_equal(raw[r][idx[r]], vals[r]), f"row {r}: value bits differ from x[idx]"
        got, want = oracle.keys(vals[r]), oracle.keys(o_vals[r])
        assert np.array_equal(got, want), f"row {r}: keys not in the oracle's order"
        same = got[1:] == got[:-1]
        assert np.all(idx[r][1:][same] > idx[r][:-1][same]), f"row {r}: equal keys not by ascending column"
        kth = want[-1]
        above = got > kth
        assert np.array_equal(idx[r][above], o_idx[r][above]), f"row {r}: entries above the k-th differ"
        if int((oracle.keys(raw[r]) >= kth).sum()) == k:
            assert np.array_equal(idx[r], o_idx[r]), f"row {r}: index order differs"


def check_stats_against_model(x, st, k, B, B2, seed, split, rows):
    for r in rows:
        res = model.row_topk(x[r], k, B, B2, seed=seed, row=r, split=split)
        want = (res.stats.W, res.stats.A, res.stats.R, res.stats.max_len)
        assert tuple(int(v) for v in st[r]) == want, f"row {r}: (W, A, R, max_len) {tuple(st[r])} != model {want}"


def plan(w):
    dt = ds.DS_F32 if w.dtype == "f32" else ds.DS_BF16
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return ds.deepselect_plan_split(dt, w.batch, w.n, w.k, w.block, w.block2, cus)


# ---------------------------------------------------------------- full-size workloads

@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_full_size(name):
    w = synth.WORKLOADS[name]
    log(f"[gpu] workload {name}: batch {w.batch} N {w.n} {w.dtype} k {w.k} B {w.block} B2 {w.block2}")
    x = synth.generate(name)
    S = plan(w)
    vals, idx, st = run_gpu(x, w.k, w.block, w.block2, seed=0, split=0)
    check_rows(x, vals, idx, w.k)
    rows = range(min(w.batch, 6))
    check_stats_against_model(x, st, w.k, w.block, w.block2, 0, S, rows)
    assert np.all(st[:, 3] <= max(w.k + w.block + w.block2 - 1, 2 * w.k + w.block2 - 1))


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_device_w_within_the_bound(name):
    # the boxed bound (the deep-dive's section "RadixSelectTopK 总处理元素数的期望上界")
    # is an expectation over the random block order: the device's W per row,
    # averaged over rows and seeds 0, 1, 2, stays at or below it (for split
    # rows the parts' bounds plus the merge's, at the library's split)
    w = synth.WORKLOADS[name]
    x = synth.generate(name)
    xt = to_device(x)
    S = plan(w)
    ws = []
    for seed in (0, 1, 2):
        out = ds.topk(xt, w.k, w.block, w.block2, seed, stats=True)
        torch.cuda.synchronize()
        ws.append(out[2].cpu().numpy()[:, 0].astype(np.float64))
    W = np.concatenate(ws)
    bound = model.expected_w_bound_row(w.n, w.k, w.block, w.block2, S)
    log(f"[gpu] W {name} split {S}: mean {W.mean():.0f} max {W.max():.0f} bound {bound:.0f} "
        f"(mean/bound {W.mean() / bound:.3f}, max/bound {W.max() / bound:.3f})")
    assert W.mean() <= bound


@pytest.mark.parametrize("name,split", [("dsa32k", 1), ("dsa32k", 2), ("dsa32k", 8),
                                        ("dsa128k_bf16", 1), ("dsa128k_bf16", 4),
                                        ("asc1m_b1", 8), ("asc1m_b1", 64), ("gauss4k", 3),
                                        ("vocab152k_k1024", 2)])
def test_forced_split(name, split):
    w = synth.WORKLOADS[name]
    rows = min(w.batch, 16)
    log(f"[gpu] forced split {name} S={split} rows {rows}")
    x = synth.generate(name, rows)
    vals, idx, st = run_gpu(x, w.k, w.block, w.block2, seed=3, split=split)
    check_rows(x, vals, idx, w.k)
    check_stats_against_model(x, st, w.k, w.block, w.block2, 3, split, range(min(rows, 4)))


@pytest.mark.parametrize("name,split,waves", [("dsa128k_bf16", 1, 4), ("dsa128k_bf16", 1, 8),
                                              ("dsa128k_bf16", 2, 8), ("dsa32k", 4, 8),
                                              ("vocab152k_k64", 1, 8), ("gauss4k", 1, 8)])
def test_forced_waves(name, split, waves):
    w = synth.WORKLOADS[name]
    rows = min(w.batch, 24)
    log(f"[gpu] forced waves {name} S={split} waves={waves} rows {rows}")
    x = synth.generate(name, rows)
    vals, idx, st = run_gpu(x, w.k, w.block, w.block2, seed=5, split=split, waves=waves)
    check_rows(x, vals, idx, w.k)
    check_stats_against_model(x, st, w.k, w.block, w.block2, 5, split, range(min(rows, 4)))


def bf16_rows_of_keys(keys: np.ndarray) -> np.ndarray:
    """bfloat16 rows (uint16 bit patterns) whose order-preserving keys are
    `keys`, all in [0x80, 0x7FFF]: negative values, key = ~pattern, down to
    negative infinity at key 0x7F (smaller keys would be NaN patterns)."""
    assert keys.min() >= 0x80 and keys.max() <= 0x7FFF
    return (0xFFFF - keys).astype(np.uint16)


# Windows of the radix select around the widths where the pass structure
# changes for 16-bit keys: the first compaction of a part has T unset, so
# its window is [0, largest key] = [0, W]; at most 255 key values take one
# 8-bit pass, 256 to 4095 one pass over a 4096-bin histogram, 4096 and more
# two 8-bit passes. `tie` puts that share of the row on a single key, so one
# bin's counter holds most of a buffer.
@pytest.mark.parametrize("W,tie,waves,split", [(255, 0.0, 8, 1), (256, 0.0, 8, 1), (256, 0.0, 4, 1),
                                               (4095, 0.0, 8, 1), (4095, 0.0, 4, 1), (4096, 0.0, 8, 1),
                                               (3000, 0.6, 8, 1), (3000, 0.6, 4, 2), (300, 0.9, 8, 2),
                                               (1000, 0.0, 4, 4)])
def test_select_windows_around_the_pass_widths(W, tie, waves, split):
    rng = np.random.default_rng(W * 131 + int(tie * 10) * 7 + waves + split)
    rows, n, k, B, B2 = 8, 16384, 512, 1024, 1024
    keys = rng.integers(0x80, W + 1, size=(rows, n))
    keys[rng.random((rows, n)) < tie] = 0x80 + (W - 0x80) // 3
    keys[:, ::97] = W  # every block holds the largest key
    x = bf16_rows_of_keys(keys)
    log(f"[gpu] select window W={W} tie={tie} waves={waves} S={split}")
    vals, idx, st = run_gpu(x, k, B, B2, seed=11, split=split, waves=waves)
    check_rows(x, vals, idx, k)
    check_stats_against_model(x, st, k, B, B2, 11, split, range(rows))


# Windows of more than 4095 key values once T is set (two 8-bit passes):
# rows with keys spread over [0x80, 0x7FFF], whose second compaction's k-th
# key lies within the top 4096 values of its window, and rows whose keys sit
# in [0x80, 3000] but for the largest key in every block, a window set by
# one far outlier with the k-th key near its bottom.
@pytest.mark.parametrize("kind,waves,split", [("spread", 8, 1), ("spread", 4, 2), ("spread", 8, 4),
                                              ("outliers", 8, 1), ("outliers", 4, 2)])
def test_select_windows_wider_than_one_pass(kind, waves, split):
    rng = np.random.default_rng(7 + waves + split + (100 if kind == "spread" else 0))
    rows, n, k, B, B2 = 8, 16384, 512, 1024, 1024
    keys = rng.integers(0x80, 0x8000 if kind == "spread" else 3001, size=(rows, n))
    keys[:, ::97] = 0x7FFF
    x = bf16_rows_of_keys(keys)
    log(f"[gpu] wide select window {kind} waves={waves} S={split}")
    vals, idx, st = run_gpu(x, k, B, B2, seed=11, split=split, waves=waves)
    check_rows(x, vals, idx, k)
    check_stats_against_model(x, st, k, B, B2, 11, split, range(rows))


KERNELS = {1: "ring", 2: "registers", 3: "generic"}


@pytest.mark.parametrize("name,split,waves,kernel", [
    (name, split, waves, kernel)
    for kernel in (1, 2, 3)
    for name, split, waves in [("dsa128k_bf16", 1, 8), ("dsa128k_bf16", 2, 4), ("dsa32k", 4, 8),
                               ("vocab152k_k1024", 1, 4), ("asc1m", 8, 8), ("ties1m", 8, 4),
                               ("gauss4k", 1, 8)]])
def test_each_kernel(name, split, waves, kernel):
    w = synth.WORKLOADS[name]
    rows = min(w.batch, 12)
    log(f"[gpu] kernel {KERNELS[kernel]} {name} S={split} waves={waves} rows {rows}")
    x = synth.generate(name, rows)
    vals, idx, st = run_gpu(x, w.k, w.block, w.block2, seed=7, split=split, waves=waves, kernel=kernel)
    check_rows(x, vals, idx, w.k)
    check_stats_against_model(x, st, w.k, w.block, w.block2, 7, split, range(min(rows, 4)))


@pytest.mark.parametrize("seed", [0, 1, 2, 2**63 + 5])
def test_seeds_and_determinism(seed):
    w = synth.WORKLOADS["dsa128k_bf16"]
    log(f"[gpu] seed {seed} on dsa128k_bf16 (16 rows)")
    x = synth.generate("dsa128k_bf16", 16)
    a = run_gpu(x, w.k, w.block, w.block2, seed=seed)
    b = run_gpu(x, w.k, w.block, w.block2, seed=seed)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
    check_rows(x, a[0], a[1], w.k)
    check_stats_against_model(x, a[2], w.k, w.block, w.block2, seed, plan(synth.Workload(
        "t", 16, w.n, w.dtype, w.k, w.block, w.block2, 0, "", "")), range(3))


# ---------------------------------------------------------------- edge cases

EDGE = [
    # (batch, N, k, B, B2, dtype, kind)
    (3, 1, 1, 1, 1, "f32", "gauss"),
    (2, 5, 5, 2, 1, "f32", "gauss"),        # k = N
    (4, 37, 1, 4, 5, "bf16", "small_ints"),  # k = 1, tiny blocks
    (3, 1000, 17, 1000, 1000, "f32", "special"),  # one block (N <= B)
    (2, 1001, 64, 256, 3, "f32", "gauss"),   # ragged last block, B2 != B
    (2, 4096, 64, 5000, 1, "bf16", "gauss"),  # N < B, B2 = 1
    (5, 3000, 100, 96, 40, "bf16", "special"),
    (2, 65536 + 3, 300, 1000, 700, "f32", "small_ints"),  # odd N: scalar loads
    (2, 12345, 2048, 2048, 2048, "bf16", "gauss"),
    (1, 200000, 1, 3072, 1, "f32", "gauss"),  # several tiles per block
    (2, 9000, 600, 7, 9, "f32", "gauss"),     # more than 1024 blocks -> split lower bound
]


@pytest.mark.parametrize("case", EDGE, ids=[f"{c[0]}x{c[1]}k{c[2]}B{c[3]}B2{c[4]}{c[5]}{c[6]}" for c in EDGE])
def test_edge_shapes(case):
    batch, n, k, B, B2, dt, kind = case
    log(f"[gpu] edge {case}")
    x = synth.random_rows(batch, n, dt, 77, kind)
    if ds.deepselect_validate(ds.DS_F32 if dt == "f32" else ds.DS_BF16, batch, n, n, k, B, B2) != 0:
        pytest.skip("shape outside the library's LDS limits")
    vals, idx, st = run_gpu(x, k, B, B2, seed=9)
    check_rows(x, vals, idx, k)


# The largest rows the library takes: N = 2^31 - 1 bfloat16 (one 4 GiB row) and
# two float32 rows of 2^29 + 4 elements (the second starts past byte 2^31).
# The background is a repeating run of negative values, and k distinct positive
# values are planted at seeded positions (both ends of the row among them), so
# by the plain definition the top k are exactly the planted entries, in the
# order of their values: a closed form the oracle's full sort would take
# minutes to reproduce at this size.
MAXROW = [("bf16", 1, (1 << 31) - 1, 2048, 2048, 2048, True),
          ("f32", 2, (1 << 29) + 4, 512, 1024, 1024, False)]


@pytest.mark.parametrize("case", MAXROW, ids=[f"{c[0]}-{c[1]}x{c[2]}" for c in MAXROW])
def test_maximum_row_length(case):
    dt, batch, n, k, B, B2, srt = case
    log(f"[gpu] maximum rows {case}")
    rng = np.random.default_rng(2024)
    tdt = torch.int16 if dt == "bf16" else torch.int32
    x = torch.empty((batch, n), dtype=tdt, device=DEV)
    step = 1 << 27
    for a in range(0, n, step):
        b = min(n, a + step)
        j = torch.arange(a, b, device=DEV, dtype=torch.int64) % 251
        if dt == "bf16":  # -1.0 (0xBF80) and the 250 bfloat16 values below it
            x[:, a:b] = (j + (0xBF80 - 65536)).to(torch.int16)
        else:  # -1 ... -251
            x[:, a:b] = (-(j + 1)).to(torch.float32).view(torch.int32)
    pos = np.empty((batch, k), dtype=np.int64)
    planted = np.empty((batch, k), dtype=np.int64)
    for r in range(batch):
        p = rng.choice(n - 2, size=k - 2, replace=False) + 1
        pos[r] = rng.permutation(np.concatenate([[0, n - 1], p]))
        if dt == "bf16":  # 1.0 (0x3F80) and the next k - 1 bfloat16 values
            planted[r] = 0x3F80 + rng.permutation(k)
        else:  # 1.0 ... k
            planted[r] = np.arange(1, k + 1, dtype=np.float32)[rng.permutation(k)].view(np.int32)
        x[r, torch.from_numpy(pos[r]).to(DEV)] = torch.from_numpy(planted[r]).to(DEV).to(tdt)
    xt = x.view(torch.bfloat16) if dt == "bf16" else x.view(torch.float32)
    vals, idx = ds.topk(xt, k, B, B2, sorted=srt)
    torch.cuda.synchronize()
    del x, xt
    got_v = raw_of(vals).astype(np.int64)
    got_i = idx.cpu().numpy().astype(np.int64)
    bits = 0xFFFF if dt == "bf16" else 0xFFFFFFFF
    for r in range(batch):
        want = dict(zip(pos[r].tolist(), (planted[r] & bits).tolist()))
        assert sorted(got_i[r].tolist()) == sorted(want), f"row {r}: index set differs from the planted one"
        assert [want[i] for i in got_i[r].tolist()] == got_v[r].tolist(), f"row {r}: value bits differ"
        if srt:  # the planted values are positive, so larger bits are larger values
            assert np.all(np.diff(got_v[r]) < 0), f"row {r}: not in descending order"


@pytest.mark.parametrize("dt,k,split", [("bf16", 301, 3), ("f32", 77, 2), ("f32", 1, 5), ("bf16", 2, 4)])
def test_split_odd_k(dt, k, split):
    # k not a multiple of 4: the parts' results and the merged row are written
    # one entry per lane (the four-at-a-time path needs k % 4 == 0)
    batch, n, B, B2 = 6, 20000, 1024, 512
    log(f"[gpu] split {split} with k {k}, {dt}")
    x = synth.random_rows(batch, n, dt, 31, "gauss")
    vals, idx, st = run_gpu(x, k, B, B2, seed=4, split=split)
    check_rows(x, vals, idx, k)
    check_stats_against_model(x, st, k, B, B2, 4, split, range(batch))


def test_all_minus_inf_and_nan_rows():
    n, k = 5000, 300
    x = np.full((4, n), 0xFF80, dtype=np.uint16)  # all -inf
    x[1, 4321] = 0x3F80
    x[2, ::7] = 0x7FC0  # +NaN above +inf
    x[3, ::5] = 0xFFC0  # -NaN below -inf
    x[3, 3::11] = 0x8000  # -0
    x[3, 4::13] = 0x0000  # +0
    log("[gpu] -inf / NaN / signed-zero rows")
    vals, idx, st = run_gpu(x, k, 512, 512)
    check_rows(x, vals, idx, k)


def test_row_stride_and_misaligned_base():
    w = synth.WORKLOADS["dsa32k"]
    x = synth.generate("dsa32k", 8)
    o_vals, o_idx = oracle.topk(x, w.k)
    big = np.zeros((8, w.n + 40), dtype=np.float32)
    big[:, 1:w.n + 1] = x  # row_stride N+40, base offset by one element
    t = torch.from_numpy(big).to(DEV)
    view = t[:, 1:w.n + 1]
    log("[gpu] strided, element-misaligned view")
    vals = torch.empty((8, w.k), dtype=torch.float32, device=DEV)
    idx = torch.empty((8, w.k), dtype=torch.int32, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    rc = ds.deepselect_topk(view.data_ptr(), ds.DS_F32, 8, w.n, w.n + 40, w.k, w.block, w.block2, 0,
                            vals.data_ptr(), idx.data_ptr(), stream)
    assert rc == 0
    torch.cuda.synchronize()
    check_rows(x, vals.cpu().numpy().view(np.uint32), idx.cpu().numpy(), w.k)


def test_non_default_stream_and_batch_zero():
    w = synth.WORKLOADS["gauss4k"]
    x = synth.generate("gauss4k")
    s = torch.cuda.Stream()
    log("[gpu] side stream")
    with torch.cuda.stream(s):
        xt = to_device(x)
        vals, idx = ds.topk(xt, w.k, w.block, w.block2)
    s.synchronize()
    check_rows(x, raw_of(vals), idx.cpu().numpy(), w.k)
    empty = torch.empty((0, 100), dtype=torch.float32, device=DEV)
    v, i = ds.topk(empty, 5, 10, 10)
    assert v.shape == (0, 5)


def test_caller_workspace():
    w = synth.WORKLOADS["dsa32k"]
    x = synth.generate("dsa32k", 16)
    xt = to_device(x)
    S = 4
    nbytes = ds.deepselect_workspace_bytes(ds.DS_F32, 16, w.n, w.k, w.block, w.block2, S)
    # no initial contents are needed
    ws = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=DEV)
    vals = torch.empty((16, w.k), dtype=torch.float32, device=DEV)
    idx = torch.empty((16, w.k), dtype=torch.int32, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    log("[gpu] caller workspace, two calls")
    for _ in range(2):
        rc = ds.deepselect_topk_ex(xt.data_ptr(), ds.DS_F32, 16, w.n, w.n, w.k, w.block, w.block2, 0,
                                   vals.data_ptr(), idx.data_ptr(), stream, split=S,
                                   workspace=ws.data_ptr(), workspace_bytes=nbytes)
        assert rc == 0
        torch.cuda.synchronize()
        check_rows(x, vals.cpu().numpy().view(np.uint32), idx.cpu().numpy(), w.k)
    rc = ds.deepselect_topk_ex(xt.data_ptr(), ds.DS_F32, 16, w.n, w.n, w.k, w.block, w.block2, 0,
                               vals.data_ptr(), idx.data_ptr(), stream, split=S,
                               workspace=ws.data_ptr(), workspace_bytes=nbytes - 1)
    assert rc == ds.DS_ERR_WORKSPACE


def test_library_workspace_across_shapes():
    # split calls of changing batch and split on one stream share its library
    # workspace: grown, reused by a smaller shape, and reused again
    w = synth.WORKLOADS["dsa32k"]
    x = synth.generate("dsa32k")
    for batch, S in [(16, 4), (64, 2), (8, 8), (64, 4), (32, 2), (64, 2), (64, 2)]:
        log(f"[gpu] library workspace: batch {batch} split {S}")
        vals, idx, st = run_gpu(x[:batch], w.k, w.block, w.block2, split=S)
        check_rows(x[:batch], vals, idx, w.k)
        check_stats_against_model(x[:batch], st, w.k, w.block, w.block2, 0, S, range(2))


# ---------------------------------------------------------------- sorted output

SORTED = [
    # (workload, rows, split, waves, kernel, k or None for the workload's)
    ("dsa128k_bf16", 6, 1, 8, 1, None),   # ring streaming, packed bfloat16 candidates
    ("dsa128k_bf16", 6, 2, 8, 0, None),   # split rows: the merge kernel sorts
    ("dsa32k", 8, 1, 8, 1, None),         # ring streaming, float32
    ("dsa32k", 8, 1, 4, 2, None),         # register streaming
    ("vocab152k_k64", 8, 0, 0, 3, None),  # generic kernel
    ("ties1m", 2, 0, 0, 0, None),         # every result ties: columns ascending
    ("asc1m_b1", 1, 0, 0, 0, None),       # one row in many parts
    ("gauss4k", 1, 1, 8, 0, 1),
    ("gauss4k", 1, 1, 8, 0, 3),
    ("gauss4k", 1, 1, 8, 0, 300),         # k not a power of two
    ("gauss4k", 1, 1, 4, 0, 4096),        # k = N
]


@pytest.mark.parametrize("case", SORTED, ids=[f"{c[0]}-S{c[2]}-w{c[3]}-kern{c[4]}-k{c[5]}" for c in SORTED])
def test_sorted_output(case):
    name, rows, split, waves, kernel, k = case
    w = synth.WORKLOADS[name]
    k = w.k if k is None else k
    log(f"[gpu] sorted output {case}")
    x = synth.generate(name, rows)
    vals, idx, st = run_gpu(x, k, w.block, w.block2, seed=3, split=split, waves=waves, kernel=kernel,
                            sorted=True)
    check_sorted_rows(x, vals, idx, k)
    # the same set and the same control flow as the unsorted call
    u_vals, u_idx, u_st = run_gpu(x, k, w.block, w.block2, seed=3, split=split, waves=waves, kernel=kernel)
    assert np.array_equal(st, u_st)
    for r in range(rows):
        assert np.array_equal(np.sort(idx[r]), np.sort(u_idx[r]))


# ---------------------------------------------------------------- per-row valid lengths

def run_gpu_len(x: np.ndarray, k, B, B2, lengths, seed=0, split=0, waves=0, kernel=0, sorted=False):
    xt = to_device(x)
    lt = torch.from_numpy(np.asarray(lengths, dtype=np.int32)).to(DEV)
    out = ds.topk(xt, k, B, B2, seed, split=split, stats=True, waves=waves, kernel=kernel, sorted=sorted,
                  lengths=lt)
    torch.cuda.synchronize()
    return raw_of(out[0]), out[1].cpu().numpy(), out[2].cpu().numpy()


def check_rows_len(x: np.ndarray, vals, idx, k, lengths, sorted=False):
    """Row r against the oracle on its prefix x[r, :L_r] (L_r clamped to
    [0, N]); outputs past min(k, L_r) are fillers (-1, negative infinity)."""
    n = x.shape[1]
    neg_inf = 0xFF800000 if x.dtype == np.float32 else 0xFF80
    for r in range(x.shape[0]):
        L = min(max(int(lengths[r]), 0), n)
        c = min(k, L)
        assert np.all(idx[r][c:] == -1), f"row {r}: filler index"
        assert np.all(vals[r][c:] == neg_inf), f"row {r}: filler value"
        if c == 0:
            continue
        sub = np.ascontiguousarray(x[r:r + 1, :L])
        if sorted:
            check_sorted_rows(sub, vals[r:r + 1, :c], idx[r:r + 1, :c], c)
        else:
            check_rows(sub, vals[r:r + 1, :c], idx[r:r + 1, :c], c)


def check_stats_len(x, st, k, B, B2, seed, split, lengths, rows):
    for r in rows:
        res = model.row_topk(x[r], k, B, B2, seed=seed, row=r, split=split, length=int(lengths[r]))
        want = (res.stats.W, res.stats.A, res.stats.R, res.stats.max_len)
        assert tuple(int(v) for v in st[r]) == want, f"row {r}: (W, A, R, max_len) {tuple(st[r])} != model {want}"


@pytest.mark.parametrize("split,waves,kernel", [(1, 8, 1), (2, 8, 1), (4, 4, 1), (2, 8, 2), (2, 4, 3)])
def test_causal_lengths(split, waves, kernel):
    # the causal rows with their valid lengths: the top-k of each prefix
    w = synth.WORKLOADS["dsa128k_bf16"]
    rows = 8
    log(f"[gpu] causal lengths dsa128k_bf16 S={split} waves={waves} kernel {KERNELS[kernel]}")
    x = synth.generate("dsa128k_bf16", rows)
    L = synth.valid_lengths("dsa128k_bf16", range(rows))
    vals, idx, st = run_gpu_len(x, w.k, w.block, w.block2, L, seed=5, split=split, waves=waves, kernel=kernel)
    check_rows_len(x, vals, idx, w.k, L)
    check_stats_len(x, st, w.k, w.block, w.block2, 5, split, L, range(4))


LEN_EDGE = [0, 1, 7, 95, 96, 97, 255, 257, 600, 515, 4999, 5000, 5050, -4]


@pytest.mark.parametrize("dt,split,kernel,srt", [("f32", 1, 0, False), ("bf16", 1, 0, False), ("f32", 3, 0, False),
                                                 ("bf16", 3, 0, True), ("f32", 2, 2, True), ("bf16", 2, 3, False),
                                                 ("f32", 1, 3, True), ("bf16", 2, 1, False), ("bf16", 2, 1, True)])
def test_edge_lengths(dt, split, kernel, srt):
    # lengths of every kind in one call: none, fewer than k, ragged inside a
    # 16-byte load, fewer blocks than parts, N, past N and negative (clamped);
    # bfloat16 in two ring parts takes the merge by the part that ends last,
    # with parts of fewer than k results, none, and no k-th key at all
    n, k, B, B2 = 5000, 96, 256, 128
    rows = len(LEN_EDGE)
    log(f"[gpu] edge lengths {dt} S={split} kernel {KERNELS.get(kernel, 'auto')} sorted={srt}")
    x = synth.random_rows(rows, n, dt, 41, "gauss")
    vals, idx, st = run_gpu_len(x, k, B, B2, LEN_EDGE, seed=3, split=split, kernel=kernel, sorted=srt)
    check_rows_len(x, vals, idx, k, LEN_EDGE, sorted=srt)
    check_stats_len(x, st, k, B, B2, 3, split, LEN_EDGE, range(rows))


def test_full_lengths_equal_the_plain_call():
    # the same result set (ties included) and statistics; the unsorted order
    # may differ where the two paths merge differently (rows of two bfloat16
    # parts are merged by the part that ends last without lengths, by the
    # merge kernel with them)
    w = synth.WORKLOADS["dsa32k"]
    x = synth.generate("dsa32k", 8)
    log("[gpu] lengths = N against no lengths")
    a = run_gpu(x, w.k, w.block, w.block2, seed=2, split=2)
    b = run_gpu_len(x, w.k, w.block, w.block2, [w.n] * 8, seed=2, split=2)
    assert np.array_equal(a[2], b[2])
    for r in range(8):
        oa, ob = np.argsort(a[1][r]), np.argsort(b[1][r])
        assert np.array_equal(a[1][r][oa], b[1][r][ob]) and np.array_equal(a[0][r][oa], b[0][r][ob])


# ---------------------------------------------------------------- fused sampling

def sample_consistent(po: np.ndarray, top_p: float, u: float, s: int, delta: float = 1e-5) -> bool:
    """Position s is a valid draw for u: the oracle's (float64) cumulative
    probabilities put u times the nucleus mass between positions s-1 and s, up
    to delta; near a boundary (of the nucleus or of a position) either side is
    accepted, since float32 may land on it."""
    c = np.cumsum(po)
    jp_o = oracle_sampling.nucleus_end(po, top_p)
    cands = {jp_o} | {j for j in range(len(po)) if abs(c[j] - top_p) <= delta}
    for jp in cands:
        if s > jp:
            continue
        target = u * c[jp]
        lo = c[s - 1] if s > 0 else 0.0
        if lo <= target + delta and (c[s] >= target - delta or s == jp):
            return True
    return False


def check_sampling(x, vals, idx, probs, sampled, k, u, temperature, top_p, lengths=None):
    n = x.shape[1]
    for r in range(x.shape[0]):
        L = n if lengths is None else min(max(int(lengths[r]), 0), n)
        c = min(k, L)
        po = np.zeros(k)
        po[:c] = oracle_sampling.softmax(oracle_sampling.values_of(vals[r][:c]), temperature)
        assert np.all(np.abs(probs[r] - po) <= 2e-5 * po + 1e-9), f"row {r}: probabilities"
        if c == 0 or po.sum() == 0.0:
            assert sampled[r] == -1
            continue
        pos = np.nonzero(idx[r][:c] == sampled[r])[0]
        assert len(pos) == 1, f"row {r}: the sampled column is not one of the results"
        assert sample_consistent(po[:c], top_p, float(u[r]), int(pos[0])), \
            f"row {r}: draw at position {int(pos[0])} does not fit u={u[r]}"


SAMPLE = [
    # (workload, rows, k or None, temperature, top_p, split)
    ("vocab152k_k64", 8, None, 1.0, 1.0, 0),
    ("vocab152k_k64", 8, None, 0.7, 0.9, 0),
    ("vocab152k_k1024", 4, None, 1.3, 0.95, 0),
    ("dsa128k_bf16", 4, 1024, 1.0, 0.8, 2),   # bfloat16, the merge kernel writes
    ("ties1m", 2, None, 1.0, 0.5, 0),         # every result ties: uniform
    ("gauss4k", 1, 1, 1.0, 1.0, 1),           # k = 1: probability 1
]


@pytest.mark.parametrize("case", SAMPLE, ids=[f"{c[0]}-k{c[2]}-t{c[3]}-p{c[4]}-S{c[5]}" for c in SAMPLE])
def test_fused_sampling(case):
    name, rows, k, temperature, top_p, split = case
    w = synth.WORKLOADS[name]
    k = w.k if k is None else k
    log(f"[gpu] fused sampling {case}")
    x = synth.generate(name, rows)
    u = np.random.default_rng(11).random(rows, dtype=np.float32)
    ut = torch.from_numpy(u).to(DEV)
    v, i, pr, sm = ds.topk_sample(to_device(x), k, w.block, w.block2, ut, seed=6, temperature=temperature,
                                  top_p=top_p, split=split)
    torch.cuda.synchronize()
    vals, idx = raw_of(v), i.cpu().numpy()
    check_sorted_rows(x, vals, idx, k)
    check_sampling(x, vals, idx, pr.cpu().numpy(), sm.cpu().numpy(), k, u, temperature, top_p)


def test_fused_sampling_short_rows():
    # rows shorter than k: probabilities over the valid results only, fillers
    # at 0, and an empty row draws -1
    n, k, B, B2 = 3000, 64, 256, 128
    lengths = [0, 1, 40, 64, 65, 3000]
    x = synth.random_rows(len(lengths), n, "bf16", 17, "gauss")
    u = np.random.default_rng(3).random(len(lengths), dtype=np.float32)
    log("[gpu] fused sampling on short rows")
    lt = torch.from_numpy(np.asarray(lengths, dtype=np.int32)).to(DEV)
    v, i, pr, sm = ds.topk_sample(to_device(x), k, B, B2, torch.from_numpy(u).to(DEV), seed=1,
                                  temperature=0.9, top_p=0.97, lengths=lt)
    torch.cuda.synchronize()
    vals, idx = raw_of(v), i.cpu().numpy()
    check_rows_len(x, vals, idx, k, lengths, sorted=True)
    check_sampling(x, vals, idx, pr.cpu().numpy(), sm.cpu().numpy(), k, u, 0.9, 0.97, lengths)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_fused_sampling_infinite_maximum(dt):
    # rows whose largest results are +inf: those share the mass equally, the
    # others get 0 (one +inf, three, none, and +inf next to -inf and NaN)
    n, k, B, B2 = 2000, 32, 256, 256
    x = synth.random_rows(4, n, dt, 23, "gauss")
    raw = x.view(np.uint32) if dt == "f32" else x  # the bit patterns, in place
    # +inf, -inf and a negative NaN (below -inf in key order)
    pinf, ninf, nnan = (0x7F800000, 0xFF800000, 0xFFC00000) if dt == "f32" else (0x7F80, 0xFF80, 0xFFC0)
    raw[0, 5] = pinf
    raw[1, [7, 700, 1999]] = pinf
    raw[3, [0, 1]] = pinf
    raw[3, 2:40] = ninf
    raw[3, 40] = nnan
    u = np.asarray([0.1, 0.5, 0.9, 0.99], dtype=np.float32)
    log(f"[gpu] fused sampling with +inf results ({dt})")
    v, i, pr, sm = ds.topk_sample(to_device(x), k, B, B2, torch.from_numpy(u).to(DEV), seed=2)
    torch.cuda.synchronize()
    vals, idx, probs = raw_of(v), i.cpu().numpy(), pr.cpu().numpy()
    check_sorted_rows(x, vals, idx, k)
    check_sampling(x, vals, idx, probs, sm.cpu().numpy(), k, u, 1.0, 1.0)
    assert probs[0, 0] == 1.0 and np.all(probs[0, 1:] == 0.0)
    assert np.allclose(probs[1, :3], 1 / 3) and np.all(probs[1, 3:] == 0.0)
    assert np.all(probs[3, :2] == 0.5) and np.all(probs[3, 2:] == 0.0)
    assert np.all(np.isfinite(probs))


# ---------------------------------------------------------------- merge: parts that cannot contribute

def skew_rows(pattern, rows, n, dt, rng):
    """Rows whose large values sit in chosen parts: ascending (only the last
    part can contribute to the merge), descending (only the first), two
    bumps (two parts), or Gaussian (every part)."""
    i = np.arange(n, dtype=np.float64)
    out = np.empty((rows, n), dtype=np.float64)
    for r in range(rows):
        noise = rng.standard_normal(n)
        if pattern == "ascending":
            out[r] = i / n * 100.0 + 1e-3 * noise
        elif pattern == "descending":
            out[r] = (n - i) / n * 100.0 + 1e-3 * noise
        elif pattern == "two_bumps":
            out[r] = noise
            out[r, n // 8: n // 8 + n // 16] += 50.0
            out[r, 6 * n // 8: 6 * n // 8 + n // 16] += 50.0
        else:
            out[r] = noise
    x = out.astype(np.float32)
    return x if dt == "f32" else synth.f32_to_bf16_bits(x)


MERGE_SKIP = [(dt, pattern, split) for dt in ("f32", "bf16") for pattern in
              ("ascending", "descending", "two_bumps", "gauss") for split in (8, 32)]


@pytest.mark.parametrize("dt,pattern,split", MERGE_SKIP, ids=[f"{c[0]}-{c[1]}-S{c[2]}" for c in MERGE_SKIP])
def test_merge_skips_parts_that_cannot_contribute(dt, pattern, split):
    # the merge counts a part whose largest key is below t0 as empty without
    # reading it, and with at most one contributing part builds no order: the
    # results and the statistics are the model's either way
    rng = np.random.default_rng(4242)
    n, k, B = 16384, 512, 256
    x = skew_rows(pattern, 2, n, dt, rng)
    log(f"[gpu] merge skip {dt} {pattern} split {split}")
    vals, idx, st = run_gpu(x, k, B, B, seed=5, split=split)
    check_rows(x, vals, idx, k)
    check_stats_against_model(x, st, k, B, B, 5, split, range(x.shape[0]))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_merge_skip_with_lengths(dt):
    # ascending rows cut short: no part with k results (t0 = 0, every part
    # with results admits), one part with results, or several
    rng = np.random.default_rng(4243)
    n, k, B, split = 16384, 512, 256, 16
    x = skew_rows("ascending", 5, n, dt, rng)
    lengths = np.asarray([100, 700, 3000, 9000, n], dtype=np.int32)
    log(f"[gpu] merge skip with lengths {dt}")
    vals, idx, st = run_gpu_len(x, k, B, B, lengths, seed=6, split=split)
    check_rows_len(x, vals, idx, k, lengths)
    check_stats_len(x, st, k, B, B, 6, split, lengths, range(x.shape[0]))


# ---------------------------------------------------------------- merge of two parts in registers

MERGE_PAIR = [
    # (dtype, k, B, B2, pattern): two parts of one merge tile each
    ("bf16", 2048, 2048, 2048, "gauss"),     # the long-context shape
    ("bf16", 2048, 2048, 512, "ties"),       # B2 < k: the merge's own compaction can trigger
    ("f32", 512, 1024, 256, "ties"),
    ("f32", 1024, 1024, 1024, "gauss"),
    ("f32", 300, 256, 100, "gauss"),         # k not a multiple of 64
    ("bf16", 1, 64, 1, "ties"),
    ("f32", 512, 1024, 1024, "ascending"),   # only the second part admits results
    ("bf16", 777, 512, 333, "descending"),   # only the first: no select in the merge
]


@pytest.mark.parametrize("dt,k,B,B2,pattern", MERGE_PAIR, ids=[f"{c[0]}-k{c[1]}-B2{c[3]}-{c[4]}" for c in MERGE_PAIR])
def test_merge_of_two_parts_in_registers(dt, k, B, B2, pattern):
    # the two-part merge runs in registers for unsorted output; with sorted
    # output, or valid lengths given (here the full rows), it takes the tile
    # loop and the candidate buffer, which keep the same results (ties
    # included): the index sets must agree row by row, and all must agree
    # with the oracle and the model's statistics
    rng = np.random.default_rng(9090)
    n, rows = 16384, 6
    if pattern == "ties":
        x32 = (rng.integers(0, 16, size=(rows, n)).astype(np.float32) * 0.5 - 3.0)
        x = x32 if dt == "f32" else synth.f32_to_bf16_bits(x32)
    else:
        x = skew_rows(pattern, rows, n, dt, rng)
    log(f"[gpu] two-part merge {dt} k {k} B {B} B2 {B2} {pattern}")
    vals, idx, st = run_gpu(x, k, B, B2, seed=9, split=2)
    check_rows(x, vals, idx, k)
    check_stats_against_model(x, st, k, B, B2, 9, 2, range(rows))
    s_vals, s_idx, s_st = run_gpu(x, k, B, B2, seed=9, split=2, sorted=True)
    check_sorted_rows(x, s_vals, s_idx, k)
    l_vals, l_idx, l_st = run_gpu_len(x, k, B, B2, np.full(rows, n, dtype=np.int32), seed=9, split=2)
    check_rows(x, l_vals, l_idx, k)
    assert np.array_equal(st, s_st) and np.array_equal(st, l_st)
    for r in range(rows):
        assert np.array_equal(np.sort(idx[r]), np.sort(s_idx[r])), f"row {r}: sorted kept set differs"
        assert np.array_equal(np.sort(idx[r]), np.sort(l_idx[r])), f"row {r}: kept set differs from the loop's"


# ---------------------------------------------------------------- shared thresholds

SHARE = [
    # (workload, rows, split, sorted, with the causal lengths)
    ("asc1m", 4, 8, False, False),
    ("asc1m_b1", 1, 16, True, False),
    ("ties1m", 4, 8, False, False),
    ("dsa32k", 8, 4, False, False),
    ("dsa128k_bf16", 8, 2, False, False),
    ("dsa128k_bf16", 8, 4, True, True),
]


@pytest.mark.parametrize("case", SHARE, ids=[f"{c[0]}-S{c[2]}-sorted{c[3]}-len{c[4]}" for c in SHARE])
def test_shared_threshold(case):
    # the result set is the plain call's; the cost is timing-dependent, but W
    # = A + k*R holds per row
    name, rows, split, srt, with_len = case
    w = synth.WORKLOADS[name]
    log(f"[gpu] shared thresholds {case}")
    x = synth.generate(name, rows)
    xt = to_device(x)
    kw = dict(split=split, stats=True, sorted=srt)
    L = None
    if with_len:
        L = synth.valid_lengths(name, range(rows))
        kw["lengths"] = torch.from_numpy(L).to(DEV)
    plain = ds.topk(xt, w.k, w.block, w.block2, 4, **kw)
    shared = ds.topk(xt, w.k, w.block, w.block2, 4, share_threshold=True, **kw)
    torch.cuda.synchronize()
    vals, idx, st = raw_of(shared[0]), shared[1].cpu().numpy(), shared[2].cpu().numpy()
    if with_len:
        check_rows_len(x, vals, idx, w.k, L, sorted=srt)
    elif srt:
        check_sorted_rows(x, vals, idx, w.k)
    else:
        check_rows(x, vals, idx, w.k)
    st0 = plain[2].cpu().numpy()
    assert np.all(st[:, 0] == st[:, 1] + w.k * st[:, 2]), "W = A + k R"
    log(f"[gpu]   admitted: {int(st0[:, 1].sum())} plain, {int(st[:, 1].sum())} shared")
    if name.startswith("asc1m"):
        # ascending rows: the top part's threshold stops the lower parts early
        assert st[:, 1].sum() <= 0.9 * st0[:, 1].sum(), "sharing did not cut the admissions"
    # the row cells are cleared by the call itself: a second call gives a
    # valid result again
    again = ds.topk(xt, w.k, w.block, w.block2, 4, share_threshold=True, **kw)
    torch.cuda.synchronize()
    if not with_len and not srt:
        check_rows(x, raw_of(again[0]), again[1].cpu().numpy(), w.k)


def check_topk_values(x, vals, idx, k):
    """Row by row: the k values are the k largest of the row as a multiset
    (np.partition), each index points at its value, no index repeats."""
    v = vals.view(np.float32)
    top = -np.sort(np.partition(-x, k - 1, axis=1)[:, :k], axis=1)
    assert np.array_equal(-np.sort(-v, axis=1), top)
    assert np.array_equal(np.take_along_axis(x, idx.astype(np.int64), axis=1), v)
    srt = np.sort(idx, axis=1)
    assert np.all(srt[:, 1:] != srt[:, :-1])


def test_shared_cells_left_zero():
    # the merge leaves every row cell zero and the library workspace's
    # reserved cells are cleared once, so a call on much smaller values right
    # after one on larger values must not be filtered by the earlier
    # thresholds (batches below and above the 1024 reserved cells, calls
    # without sharing in between). Rows ascend, so the upper part's threshold
    # stops the lower part once it arrives: the admissions over the sequence
    # show that the sharing path ran. (65536 columns in blocks of 512, two
    # parts: 8 ring steps per wave, or 16 on the 1100-row calls.)
    n, k, B, B2, S = 65536, 64, 512, 512, 2
    seq = [(3, 1000.0, True), (5, 0.0, True), (1, 5000.0, False), (1100, 2000.0, True), (1100, -10.0, True),
           (2, -3000.0, True), (6, -4000.0, True)]
    a_plain = a_shared = 0
    for rows, shift, share in seq:
        log(f"[gpu] shared cells: rows {rows} shift {shift} share {share}")
        ramp = np.float32(shift) + np.arange(n, dtype=np.float32) * np.float32(100.0 / n)
        x = np.tile(ramp, (rows, 1))
        xt = to_device(x)
        if share:
            _, _, st0 = ds.topk(xt, k, B, B2, 11, split=S, stats=True)
        v, i, st = ds.topk(xt, k, B, B2, 11, split=S, stats=True, share_threshold=share)
        torch.cuda.synchronize()
        check_topk_values(x, raw_of(v), i.cpu().numpy(), k)
        st = st.cpu().numpy()
        assert np.all(st[:, 0] == st[:, 1] + k * st[:, 2]), "W = A + k R"
        if share:
            a_plain += int(st0.cpu().numpy()[:, 1].sum())
            a_shared += int(st[:, 1].sum())
    log(f"[gpu]   admitted over the shared calls: {a_plain} plain, {a_shared} shared")
    assert a_shared < a_plain, "the parts did not share thresholds"


# ---------------------------------------------------------------- randomised parity

def draw_case(i):
    """Seeded draw of one call: dtype, shape, values, k, B, B2, split, waves,
    kernel, sorted output and valid lengths (redrawn until the library takes
    the shape and the method model stays quick)."""
    rng = np.random.default_rng(7000 + i)
    while True:
        dt = str(rng.choice(["f32", "bf16"]))
        batch = int(rng.integers(1, 7))
        n = max(1, int(np.exp(rng.uniform(0.0, np.log(40000.0)))))
        k = max(1, int(np.exp(rng.uniform(0.0, np.log(min(n, 2500))))))
        B = max(1, int(np.exp(rng.uniform(0.0, np.log(4096.0)))))
        B2 = max(1, int(np.exp(rng.uniform(0.0, np.log(4096.0)))))
        dcode = ds.DS_F32 if dt == "f32" else ds.DS_BF16
        if ds.deepselect_validate(dcode, batch, n, n, k, B, B2) != 0 or -(-n // B) > 3000:
            continue
        lengths = rng.integers(-2, n + 3, batch) if rng.random() < 0.3 else None
        return dict(dt=dt, batch=batch, n=n, k=k, B=B, B2=B2, kind=str(rng.choice(["gauss", "small_ints", "special"])),
                    split=int(rng.choice([0, 0, 1, 2, 3, 5])), waves=int(rng.choice([0, 4, 8])),
                    kernel=int(rng.choice([0, 0, 1, 2, 3])), sorted=bool(rng.integers(2)), lengths=lengths,
                    seed=int(rng.integers(0, 2**63, dtype=np.uint64)), data=int(rng.integers(1 << 30)))


@pytest.mark.parametrize("i", range(150))
def test_random_calls(i):
    c = draw_case(i)
    log(f"[gpu] random call {i}: " + ", ".join(f"{a}={c[a]}" for a in ("dt", "batch", "n", "k", "B", "B2", "kind",
                                                                        "split", "waves", "kernel", "sorted")))
    x = synth.random_rows(c["batch"], c["n"], c["dt"], c["data"], c["kind"])
    xt = to_device(x)
    lt = None if c["lengths"] is None else torch.from_numpy(c["lengths"].astype(np.int32)).to(DEV)
    split, waves, kernel = c["split"], c["waves"], c["kernel"]
    # a quarter of the calls also share thresholds between the parts of a
    # row (drawn apart, so the draws above stay as they are)
    share = bool(np.random.default_rng(9000 + i).random() < 0.25)
    try:
        out = ds.topk(xt, c["k"], c["B"], c["B2"], c["seed"], split=split, stats=True, waves=waves, kernel=kernel,
                      sorted=c["sorted"], lengths=lt, share_threshold=share)
    except ds.DeepSelectArgumentError:
        # a forced split, wave count or kernel this shape does not allow: the
        # library's own choice must take it
        assert (split, waves, kernel) != (0, 0, 0)
        log(f"[gpu]   split={split} waves={waves} kernel={kernel} refused for this shape; library choice")
        split, waves, kernel = 0, 0, 0
        out = ds.topk(xt, c["k"], c["B"], c["B2"], c["seed"], stats=True, sorted=c["sorted"], lengths=lt,
                      share_threshold=share)
    torch.cuda.synchronize()
    vals, idx, st = raw_of(out[0]), out[1].cpu().numpy(), out[2].cpu().numpy()
    n, k = c["n"], c["k"]
    lengths = c["lengths"] if c["lengths"] is not None else np.full(c["batch"], n)
    check_rows_len(x, vals, idx, k, lengths, sorted=c["sorted"])
    if share:
        log("[gpu]   shared thresholds: the cost depends on timing, the result may not")
        return
    if split == 0:
        dcode = ds.DS_F32 if c["dt"] == "f32" else ds.DS_BF16
        split = ds.deepselect_plan_split(dcode, c["batch"], n, k, c["B"], c["B2"],
                                         torch.cuda.get_device_properties(0).multi_processor_count)
    check_stats_len(x, st, k, c["B"], c["B2"], c["seed"], split, lengths, range(min(2, c["batch"])))


# ---------------------------------------------------------------- HIP graph capture

@pytest.mark.parametrize("share", [False, True])
def test_graph_capture_replays(share):
    # a call with a caller workspace launches kernels only (no allocation, no
    # memset), so it can be captured in a HIP graph; every replay, with other
    # work and synchronisations between them, must give the eager result
    w = synth.WORKLOADS["dsa32k"]
    rows, S = 16, 4
    log(f"[gpu] graph capture, split {S}, shared thresholds {share}")
    x = synth.generate("dsa32k", rows)
    xt = to_device(x)
    other = to_device(synth.random_rows(rows, w.n, "f32", 5, "gauss"))
    nbytes = ds.deepselect_workspace_bytes(ds.DS_F32, rows, w.n, w.k, w.block, w.block2, S)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    vals = torch.empty((rows, w.k), dtype=torch.float32, device=DEV)
    idx = torch.empty((rows, w.k), dtype=torch.int32, device=DEV)
    st = torch.empty((rows, 4), dtype=torch.int64, device=DEV)
    o_vals = torch.empty_like(vals)
    o_idx = torch.empty_like(idx)

    def call(src, v, i, stream):
        rc = ds.deepselect_topk_ex(src.data_ptr(), ds.DS_F32, rows, w.n, w.n, w.k, w.block, w.block2, 3,
                                   v.data_ptr(), i.data_ptr(), stream, split=S, stats=st.data_ptr(),
                                   workspace=ws.data_ptr(), workspace_bytes=nbytes, sorted=1,
                                   share_threshold=int(share))
        assert rc == 0, ds.deepselect_status_string(rc)

    cur = torch.cuda.current_stream().cuda_stream
    call(xt, vals, idx, cur)
    torch.cuda.synchronize()
    ref_v, ref_i, ref_st = vals.clone(), idx.clone(), st.clone()
    check_sorted_rows(x, raw_of(ref_v), ref_i.cpu().numpy(), w.k)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(xt, vals, idx, side.cuda_stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call(xt, vals, idx, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for rep in range(4):
        vals.zero_()
        idx.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(vals, ref_v) and torch.equal(idx, ref_i), f"replay {rep} differs from the eager call"
        if not share:  # with sharing the cost depends on timing
            assert torch.equal(st, ref_st), f"replay {rep}: statistics differ"
        # the program's own eager work between replays, on the same workspace
        call(other, o_vals, o_idx, cur)
        torch.cuda.synchronize()


def test_merge_in_part_kernel_repeats_and_graph_replays():
    # rows of two packed bfloat16 parts (unsorted) are merged by the part
    # that ends last, after an arrival count in the row's cell that this part
    # resets: repeated calls through the library workspace (batches on both
    # sides), calls with a caller workspace and replays of a captured graph
    # must give the first call's results and statistics, which match the
    # oracle and the model
    w = synth.WORKLOADS["dsa128k_bf16"]
    rows, S, seed = 8, 2, 4
    log(f"[gpu] merge in the part kernel: {rows} rows, split {S}")
    x = synth.generate("dsa128k_bf16", rows)
    vals, idx, st = run_gpu(x, w.k, w.block, w.block2, seed=seed, split=S)
    check_rows(x, vals, idx, w.k)
    check_stats_against_model(x, st, w.k, w.block, w.block2, seed, S, range(4))
    for rep in range(3):
        v3, i3, s3 = run_gpu(x[:3], w.k, w.block, w.block2, seed=seed, split=S)
        assert np.array_equal(v3, vals[:3]) and np.array_equal(i3, idx[:3]) and np.array_equal(s3, st[:3])
        v8, i8, s8 = run_gpu(x, w.k, w.block, w.block2, seed=seed, split=S)
        assert np.array_equal(v8, vals) and np.array_equal(i8, idx) and np.array_equal(s8, st), f"repeat {rep}"
    # a caller workspace, eagerly and captured
    xt = to_device(x)
    other = to_device(synth.generate("dsa128k_bf16", rows)[::-1].copy())
    nbytes = ds.deepselect_workspace_bytes(ds.DS_BF16, rows, w.n, w.k, w.block, w.block2, S)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    gv = torch.empty((rows, w.k), dtype=torch.bfloat16, device=DEV)
    gi = torch.empty((rows, w.k), dtype=torch.int32, device=DEV)
    gs = torch.empty((rows, 4), dtype=torch.int64, device=DEV)
    ov, oi = torch.empty_like(gv), torch.empty_like(gi)

    def call(src, v, i, stream):
        rc = ds.deepselect_topk_ex(src.data_ptr(), ds.DS_BF16, rows, w.n, w.n, w.k, w.block, w.block2, seed,
                                   v.data_ptr(), i.data_ptr(), stream, split=S, stats=gs.data_ptr(),
                                   workspace=ws.data_ptr(), workspace_bytes=nbytes)
        assert rc == 0, ds.deepselect_status_string(rc)

    cur = torch.cuda.current_stream().cuda_stream
    call(xt, gv, gi, cur)
    torch.cuda.synchronize()
    assert np.array_equal(raw_of(gv), vals) and np.array_equal(gi.cpu().numpy(), idx)
    assert np.array_equal(gs.cpu().numpy(), st)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(xt, gv, gi, side.cuda_stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call(xt, gv, gi, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for rep in range(4):
        gv.zero_()
        gi.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(raw_of(gv), vals) and np.array_equal(gi.cpu().numpy(), idx), f"replay {rep}"
        assert np.array_equal(gs.cpu().numpy(), st), f"replay {rep}: statistics differ"
        call(other, ov, oi, cur)
        torch.cuda.synchronize()


@pytest.mark.parametrize("rows,n,k,waves", [(1100, 8192, 256, 8), (40, 16384, 512, 4), (40, 16384, 1536, 8)])
def test_merge_in_part_kernel_shapes(rows, n, k, waves):
    # rows of two bfloat16 parts merged by their last part: more rows than
    # the 1024 reserved cells (the rest cleared by the small kernel each
    # call), and workgroups of 4 and 8 waves; twice in a row, against the
    # oracle and the model
    rng = np.random.default_rng(rows + k)
    x = synth.f32_to_bf16_bits(rng.standard_normal((rows, n)).astype(np.float32))
    B = 512
    log(f"[gpu] merge in the part kernel: {rows} rows x {n}, k {k}, {waves} waves")
    first = None
    for rep in range(2):
        vals, idx, st = run_gpu(x, k, B, B, seed=11, split=2, waves=waves)
        if first is None:
            check_rows(x, vals, idx, k)
            check_stats_against_model(x, st, k, B, B, 11, 2, range(0, rows, max(1, rows // 4)))
            first = (vals, idx, st)
        else:
            assert all(np.array_equal(a, b) for a, b in zip(first, (vals, idx, st))), "second call differs"


def test_two_streams_at_once():
    # split calls on two streams in flight together: each stream has its own
    # library workspace, so neither call sees the other's partial results
    w = synth.WORKLOADS["dsa32k"]
    rows = 12
    log("[gpu] two streams, split rows, library workspaces")
    xa = synth.generate("dsa32k", rows)
    xb = synth.random_rows(rows, w.n, "f32", 9, "small_ints")
    ta, tb = to_device(xa), to_device(xb)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    outs = []
    for rep in range(3):
        with torch.cuda.stream(sa):
            ra = ds.topk(ta, w.k, w.block, w.block2, split=4)
        with torch.cuda.stream(sb):
            rb = ds.topk(tb, w.k, w.block, w.block2, split=3)
        outs.append((ra, rb))
    torch.cuda.synchronize()
    for ra, rb in outs:
        check_rows(xa, raw_of(ra[0]), ra[1].cpu().numpy(), w.k)
        check_rows(xb, raw_of(rb[0]), rb[1].cpu().numpy(), w.k)


def test_two_streams_merging_in_the_part_kernel():
    # rows of two bfloat16 parts merged by their last part, on two streams in
    # flight together: each stream's library workspace has its own cells
    w = synth.WORKLOADS["dsa128k_bf16"]
    rows = 8
    log("[gpu] two streams, rows merged in the part kernel")
    xa = synth.generate("dsa128k_bf16", rows)
    xb = synth.random_rows(rows, w.n, "bf16", 10, "small_ints")
    ta, tb = to_device(xa), to_device(xb)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    outs = []
    for rep in range(3):
        with torch.cuda.stream(sa):
            ra = ds.topk(ta, w.k, w.block, w.block2, split=2)
        with torch.cuda.stream(sb):
            rb = ds.topk(tb, w.k, w.block, w.block2, split=2)
        outs.append((ra, rb))
    torch.cuda.synchronize()
    for ra, rb in outs:
        check_rows(xa, raw_of(ra[0]), ra[1].cpu().numpy(), w.k)
        check_rows(xb, raw_of(rb[0]), rb[1].cpu().numpy(), w.k)
