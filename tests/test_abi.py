"""The C-ABI library: it loads without a GPU, exports every declared entry point,
and its pure-host functions (validation, split plan, sizes) behave as the header
says. No compute call is made here."""
import math
import os
import re

import pytest

import synth
import top_selection_row_amd as ds

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "deepselect.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(deepselect_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ds.library()
    names = declared_functions()
    assert set(names) == set(ds.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


@pytest.mark.parametrize("args,status", [
    ((ds.DS_F32, 4, 100, 100, 10, 32, 32), ds.DS_OK),
    ((7, 4, 100, 100, 10, 32, 32), ds.DS_ERR_DTYPE),
    ((ds.DS_F32, -1, 100, 100, 10, 32, 32), ds.DS_ERR_SHAPE),
    ((ds.DS_F32, 4, 0, 100, 10, 32, 32), ds.DS_ERR_SHAPE),
    ((ds.DS_F32, 4, 100, 99, 10, 32, 32), ds.DS_ERR_SHAPE),
    ((ds.DS_F32, 4, 1 << 31, 1 << 31, 10, 32, 32), ds.DS_ERR_SHAPE),
    ((ds.DS_F32, 4, 100, 100, 0, 32, 32), ds.DS_ERR_K),
    ((ds.DS_F32, 4, 100, 100, 101, 32, 32), ds.DS_ERR_K),
    ((ds.DS_F32, 4, 100, 100, 10, 0, 32), ds.DS_ERR_BLOCK),
    ((ds.DS_F32, 4, 100, 100, 10, 32, 0), ds.DS_ERR_BLOCK),
    ((ds.DS_BF16, 4, 1 << 20, 1 << 20, 10000, 10000, 10000), ds.DS_ERR_UNSUPPORTED),
    ((ds.DS_BF16, 0, 100, 100, 10, 32, 32), ds.DS_OK),
])
def test_validate(args, status):
    assert ds.deepselect_validate(*args) == status


def test_topk_rejects_before_any_hip_call():
    # argument errors come back without touching a device (none exists here)
    assert ds.deepselect_topk(0, ds.DS_F32, 2, 64, 64, 8, 16, 16, 0, 0, 0, 0) == ds.DS_ERR_NULL
    assert ds.deepselect_topk(16, ds.DS_F32, 2, 64, 64, 65, 16, 16, 0, 16, 16, 0) == ds.DS_ERR_K
    assert ds.deepselect_topk(16, 5, 2, 64, 64, 8, 16, 16, 0, 16, 16, 0) == ds.DS_ERR_DTYPE
    assert ds.deepselect_topk(0, ds.DS_F32, 0, 64, 64, 8, 16, 16, 0, 0, 0, 0) == ds.DS_OK
    # element-misaligned x
    assert ds.deepselect_topk(18, ds.DS_F32, 2, 64, 64, 8, 16, 16, 0, 16, 16, 0) == ds.DS_ERR_SHAPE


def test_topk_ex_rejects_bad_options_before_any_hip_call():
    # the options are checked with the other arguments, before the device is
    # queried (none exists here, so reaching it would give DS_ERR_HIP)
    args = (16, ds.DS_F32, 2, 64, 64, 8, 16, 16, 0, 16, 16, 0)
    assert ds.deepselect_topk_ex(*args, waves=5) == ds.DS_ERR_BLOCK
    assert ds.deepselect_topk_ex(*args, kernel=4) == ds.DS_ERR_BLOCK
    assert ds.deepselect_topk_ex(*args, kernel=-1) == ds.DS_ERR_BLOCK
    assert ds.deepselect_topk_ex(*args, sorted=2) == ds.DS_ERR_BLOCK
    assert ds.deepselect_topk_ex(*args, sorted=-1) == ds.DS_ERR_BLOCK
    assert ds.deepselect_topk_ex(*args, share_threshold=2) == ds.DS_ERR_BLOCK
    # fused sampling: sorted output only, a draw needs somewhere to go, the
    # temperature and top_p in range, k within one register sort
    assert ds.deepselect_topk_ex(*args, probs=16) == ds.DS_ERR_BLOCK
    assert ds.deepselect_topk_ex(*args, sorted=1, sample_u=16) == ds.DS_ERR_NULL
    for t, p in [(-1.0, 1.0), (float("inf"), 1.0), (float("nan"), 1.0), (1.0, 1.5), (1.0, -0.1),
                 (1.0, float("nan"))]:
        assert ds.deepselect_topk_ex(*args, sorted=1, probs=16, temperature=t, top_p=p) == ds.DS_ERR_BLOCK
    big = (16, ds.DS_F32, 2, 4096, 4096, 1025, 256, 256, 0, 16, 16, 0)
    assert ds.deepselect_topk_ex(*big, sorted=1, probs=16) == ds.DS_ERR_UNSUPPORTED


def test_options_struct_matches_the_header(tmp_path):
    # the binding's ds_options_t against the C compiler's reading of the header
    import ctypes
    import pathlib
    import subprocess
    names = [f[0] for f in ds.DsOptions._fields_]
    inc = pathlib.Path(__file__).resolve().parents[1] / "include"
    src = tmp_path / "opt.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"deepselect.h\"\n"
                   "int main(void) { printf(\"%zu\", sizeof(ds_options_t));"
                   + "".join(f' printf(" %zu", offsetof(ds_options_t, {n}));' for n in names)
                   + " return 0; }\n")
    exe = tmp_path / "opt"
    subprocess.run(["gcc", "-I", str(inc), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    assert got[0] == ctypes.sizeof(ds.DsOptions)
    assert got[1:] == [getattr(ds.DsOptions, n).offset for n in names]


def test_status_strings():
    for st in range(0, -9, -1):
        s = ds.deepselect_status_string(st)
        assert s and s != "unknown status"
    assert ds.deepselect_status_string(-99) == "unknown status"


def _parts_ok(n, k, B, S):
    m = -(-n // B)
    for s in range(S):
        b0, b1 = s * m // S, (s + 1) * m // S
        if min(b1 * B, n) - b0 * B < k:
            return False
    return True


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_split_plan_is_valid(name):
    w = synth.WORKLOADS[name]
    dt = ds.DS_F32 if w.dtype == "f32" else ds.DS_BF16
    S = ds.deepselect_plan_split(dt, w.batch, w.n, w.k, w.block, w.block2, 256)
    assert S >= 1
    if S > 1:
        assert _parts_ok(w.n, w.k, w.block, S)
        assert ds.deepselect_workspace_bytes(dt, w.batch, w.n, w.k, w.block, w.block2, S) >= \
            w.batch * S * w.k * 8 + w.batch * 4
    lds = ds.deepselect_lds_bytes(dt, w.n, w.k, w.block, w.block2, S)
    L = w.k + w.block + w.block2 - 1
    assert L * (w.elem_bytes + 4) <= lds <= 160 * 1024
    # small batches are split towards one part per compute unit, within the
    # planner's caps (balance of bytes to results, four 8-block steps per part
    # or two for batches under a sixteenth of the units, at most 64 parts)
    if w.batch <= 128:
        min_blocks = 16 if w.batch * 16 <= 256 else 32
        cap = min(math.floor(math.sqrt(w.n * w.elem_bytes / (2 * w.k))), max(1, -(-w.n // w.block) // min_blocks),
                  64)
        assert S == max(1, min(-(-256 // w.batch), cap))


def test_split_plan_examples():
    assert ds.deepselect_plan_split(ds.DS_BF16, 128, 131072, 2048, 2048, 2048, 256) == 2
    assert ds.deepselect_plan_split(ds.DS_F32, 64, 32768, 512, 1024, 1024, 256) == 1
    assert ds.deepselect_plan_split(ds.DS_F32, 256, 151936, 64, 1024, 1024, 256) == 1
    assert ds.deepselect_plan_split(ds.DS_F32, 32, 1 << 20, 512, 1024, 1024, 256) == 8
    assert ds.deepselect_plan_split(ds.DS_F32, 1, 1 << 20, 512, 1024, 1024, 256) == 64
    assert ds.deepselect_plan_split(ds.DS_F32, 1, 4096, 64, 256, 256, 256) == 1


def test_workspace_layout():
    # k (key, column) pairs per part plus four statistics per part
    nbytes = ds.deepselect_workspace_bytes(ds.DS_BF16, 128, 131072, 2048, 2048, 2048, 2)
    assert nbytes >= 128 * 2 * 2048 * 8 + 128 * 2 * 32


def test_workspace_zero_without_split():
    assert ds.deepselect_workspace_bytes(ds.DS_F32, 8, 1000, 10, 100, 100, 1) == 0
    assert ds.deepselect_workspace_bytes(ds.DS_F32, 8, 1000, 0, 100, 100, 2) == 0


def test_bench_refuses_more_than_one_gpu():
    # one GPU is measured; a request for more exits with a message before any
    # device work
    import pathlib
    import subprocess
    import sys

    root = pathlib.Path(__file__).resolve().parents[1]
    r = subprocess.run([sys.executable, str(root / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_caller_outputs_are_checked():
    # topk(out=...) hands the caller's tensors to the kernels, which write
    # batch*k entries through them: shape, dtype, device and layout are checked
    import torch

    x = torch.zeros((3, 100), dtype=torch.bfloat16)
    good = (torch.empty((3, 8), dtype=torch.bfloat16), torch.empty((3, 8), dtype=torch.int32))
    assert ds._out_pair(good, x, 3, 8) == good
    bad = [
        (torch.empty((3, 7), dtype=torch.bfloat16), good[1]),               # too short
        (good[0], torch.empty((2, 8), dtype=torch.int32)),                  # too few rows
        (torch.empty((3, 8), dtype=torch.float32), good[1]),                # wrong value dtype
        (good[0], torch.empty((3, 8), dtype=torch.int64)),                  # wrong index dtype
        (torch.empty((8, 3), dtype=torch.bfloat16).t(), good[1]),           # strided
        (good[0], torch.empty((3, 16), dtype=torch.int32)[:, ::2]),         # strided
        (good[0],),                                                         # not a pair
        None,
    ]
    for out in bad:
        with pytest.raises(ValueError):
            ds._out_pair(out, x, 3, 8)
