"""Python binding of the MI355X DeepSelect row-wise top-k library (``libdeepselect.so``).

Argument marshalling only: every step of the computation runs in the HIP
library. The functions named like the C ABI in ``include/deepselect.h`` take
the same arguments (device pointers as integers, the stream as an integer
``hipStream_t``); :func:`topk` is the torch-tensor convenience wrapper, which
uses torch only to allocate outputs and to name the current stream.

There is no fallback: if the library is missing or cannot load, importing the
wrappers raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdeepselect.so")

DS_F32, DS_BF16 = 0, 1
DS_OK = 0
DS_ERR_NULL, DS_ERR_DTYPE, DS_ERR_SHAPE, DS_ERR_K = -1, -2, -3, -4
DS_ERR_BLOCK, DS_ERR_UNSUPPORTED, DS_ERR_HIP, DS_ERR_WORKSPACE, DS_ERR_SCRATCH = -5, -6, -7, -8, -9
DS_STATS_PER_ROW = 4
STAT_NAMES = ("W", "A", "R", "max_len")

EXPORTS = (
    "deepselect_validate", "deepselect_topk", "deepselect_topk_ex", "deepselect_plan_split",
    "deepselect_workspace_bytes", "deepselect_lds_bytes", "deepselect_status_string",
    "deepselect_release", "deepselect_topk_noalloc", "deepselect_scratch_bytes",
)


class DsOptions(ctypes.Structure):
    _fields_ = [("split", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("stats", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("kernel", ctypes.c_int32),
                ("sorted", ctypes.c_int32), ("lengths", ctypes.c_void_p),
                ("probs", ctypes.c_void_p), ("temperature", ctypes.c_float), ("top_p", ctypes.c_float),
                ("sample_u", ctypes.c_void_p), ("sample_idx", ctypes.c_void_p),
                ("share_threshold", ctypes.c_int32)]


_lib = None


def library() -> ctypes.CDLL:
    """Load libdeepselect.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with `python -m top_selection_row_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, vp, u64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_uint64
    lib.deepselect_validate.argtypes = [ctypes.c_int, i64, i64, i64, i32, i32, i32]
    lib.deepselect_validate.restype = ctypes.c_int
    lib.deepselect_topk.argtypes = [vp, ctypes.c_int, i64, i64, i64, i32, i32, i32, u64, vp, vp, vp]
    lib.deepselect_topk.restype = ctypes.c_int
    lib.deepselect_topk_ex.argtypes = [vp, ctypes.c_int, i64, i64, i64, i32, i32, i32, u64, vp, vp, vp,
                                       ctypes.POINTER(DsOptions)]
    lib.deepselect_topk_ex.restype = ctypes.c_int
    lib.deepselect_plan_split.argtypes = [ctypes.c_int, i64, i64, i32, i32, i32, i32]
    lib.deepselect_plan_split.restype = ctypes.c_int
    lib.deepselect_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i32, i32, i32, i32]
    lib.deepselect_workspace_bytes.restype = ctypes.c_size_t
    lib.deepselect_lds_bytes.argtypes = [ctypes.c_int, i64, i32, i32, i32, i32]
    lib.deepselect_lds_bytes.restype = ctypes.c_size_t
    lib.deepselect_status_string.argtypes = [ctypes.c_int]
    lib.deepselect_status_string.restype = ctypes.c_char_p
    lib.deepselect_release.argtypes = []
    lib.deepselect_release.restype = None
    lib.deepselect_topk_noalloc.argtypes = [vp, ctypes.c_int, i64, i64, i64, i32, i32, i32, u64, vp, vp, vp,
                                            ctypes.POINTER(DsOptions)]
    lib.deepselect_topk_noalloc.restype = ctypes.c_int
    lib.deepselect_scratch_bytes.argtypes = []
    lib.deepselect_scratch_bytes.restype = ctypes.c_size_t
    _lib = lib
    return lib


class DeepSelectError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"deepselect status {status}: {deepselect_status_string(status)}")


class DeepSelectArgumentError(DeepSelectError, ValueError):
    pass


def _check(status: int) -> int:
    if status < 0:
        if status in (DS_ERR_HIP,):
            raise DeepSelectError(status)
        raise DeepSelectArgumentError(status)
    return status


# ---------------------------------------------------------------- C-ABI names

def deepselect_status_string(status: int) -> str:
    return library().deepselect_status_string(int(status)).decode()


def deepselect_validate(dtype, batch, n, row_stride, k, B, B2) -> int:
    return library().deepselect_validate(dtype, batch, n, row_stride, k, B, B2)


def deepselect_plan_split(dtype, batch, n, k, B, B2, num_cus) -> int:
    return library().deepselect_plan_split(dtype, batch, n, k, B, B2, num_cus)


def deepselect_workspace_bytes(dtype, batch, n, k, B, B2, split) -> int:
    return library().deepselect_workspace_bytes(dtype, batch, n, k, B, B2, split)


def deepselect_lds_bytes(dtype, n, k, B, B2, split) -> int:
    return library().deepselect_lds_bytes(dtype, n, k, B, B2, split)


def deepselect_release() -> None:
    library().deepselect_release()


def deepselect_topk(x, dtype, batch, n, row_stride, k, B, B2, seed, out_vals, out_idx, stream) -> int:
    return library().deepselect_topk(x, dtype, batch, n, row_stride, k, B, B2, seed & (2**64 - 1),
                                     out_vals, out_idx, stream)


def deepselect_topk_ex(x, dtype, batch, n, row_stride, k, B, B2, seed, out_vals, out_idx, stream,
                       split=0, stats=None, workspace=None, workspace_bytes=0, waves=0, kernel=0,
                       sorted=0, lengths=None, probs=None, temperature=0.0, top_p=0.0, sample_u=None,
                       sample_idx=None, share_threshold=0) -> int:
    opt = DsOptions(int(split), int(waves), stats, workspace, int(workspace_bytes), int(kernel), int(sorted),
                    lengths, probs, float(temperature), float(top_p), sample_u, sample_idx, int(share_threshold))
    return library().deepselect_topk_ex(x, dtype, batch, n, row_stride, k, B, B2, seed & (2**64 - 1),
                                        out_vals, out_idx, stream, ctypes.byref(opt))


def deepselect_topk_noalloc(x, dtype, batch, n, row_stride, k, B, B2, seed, out_vals, out_idx, stream,
                            split=0, stats=None, waves=0, kernel=0, sorted=0, lengths=None, probs=None,
                            temperature=0.0, top_p=0.0, sample_u=None, sample_idx=None,
                            share_threshold=0) -> int:
    opt = DsOptions(int(split), int(waves), stats, None, 0, int(kernel), int(sorted), lengths, probs,
                    float(temperature), float(top_p), sample_u, sample_idx, int(share_threshold))
    return library().deepselect_topk_noalloc(x, dtype, batch, n, row_stride, k, B, B2, seed & (2**64 - 1),
                                             out_vals, out_idx, stream, ctypes.byref(opt))


def deepselect_scratch_bytes() -> int:
    return library().deepselect_scratch_bytes()


# ---------------------------------------------------------------- torch wrapper

def _lengths_ptr(lengths, x, batch):
    if lengths is None:
        return None
    import torch

    if (lengths.dtype != torch.int32 or lengths.device != x.device or lengths.dim() != 1
            or lengths.shape[0] != batch or not lengths.is_contiguous()):
        raise ValueError("lengths must be a contiguous int32 tensor of batch entries on x's device")
    return lengths.data_ptr()


def _out_pair(out, x, batch, k):
    """Check caller-given outputs: (vals, idx) of shape (batch, k), contiguous,
    vals in x's dtype and idx int32, both on x's device. The kernels write
    batch*k entries through them, so anything else is refused."""
    import torch

    try:
        vals, idx = out
    except (TypeError, ValueError):
        raise ValueError("out must be a pair (vals, idx)") from None
    for t, dt, name in ((vals, x.dtype, "vals"), (idx, torch.int32, "idx")):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"out {name} must be a tensor")
        if tuple(t.shape) != (batch, k) or t.dtype != dt or t.device != x.device or not t.is_contiguous():
            raise ValueError(f"out {name} must be a contiguous ({batch}, {k}) {dt} tensor on {x.device}, "
                             f"got {tuple(t.shape)} {t.dtype} on {t.device}")
    return vals, idx


def topk(x, k: int, B: int, B2: int, seed: int = 0, *, split: int = 0, waves: int = 0,
         kernel: int = 0, stats: bool = False, sorted: bool = False, lengths=None, share_threshold: bool = False,
         out=None, stream=None):
    """Row-wise top-k of a 2-D CUDA tensor (float32 or bfloat16, unit column stride).

    ``kernel``: 0 library choice, 1 ring streaming, 2 register streaming,
    3 generic (``ds_options_t.kernel`` of the C header).

    Returns (vals [batch, k] same dtype, idx [batch, k] int32) and, with
    ``stats=True``, a [batch, 4] int64 tensor (W, A, R, max_len). The k entries
    of a row are in no particular order, or with ``sorted=True`` largest first
    (equal values by ascending column). ``lengths``: an optional int32 device
    tensor of ``batch`` valid row lengths (``ds_options_t.lengths``: row r is
    its first lengths[r] elements; outputs past a row shorter than k are index
    -1 with value -inf). ``out``: an optional (vals, idx) pair to write into,
    contiguous (batch, k) tensors of x's dtype and int32 on x's device. Raises
    on any rejected argument.
    """
    import torch

    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D tensor with unit stride along the row")
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    if x.dtype == torch.float32:
        dt = DS_F32
    elif x.dtype == torch.bfloat16:
        dt = DS_BF16
    else:
        raise ValueError(f"unsupported dtype {x.dtype}")
    batch, n = x.shape
    row_stride = x.stride(0) if batch > 1 else n
    if out is None:
        vals = torch.empty((batch, k), dtype=x.dtype, device=x.device)
        idx = torch.empty((batch, k), dtype=torch.int32, device=x.device)
    else:
        vals, idx = _out_pair(out, x, batch, k)
    st = torch.empty((batch, DS_STATS_PER_ROW), dtype=torch.int64, device=x.device) if stats else None
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    with torch.cuda.device(x.device):
        _check(deepselect_topk_ex(x.data_ptr(), dt, batch, n, row_stride, k, B, B2, seed,
                                  vals.data_ptr(), idx.data_ptr(), stream, split=split, waves=waves,
                                  kernel=kernel, stats=st.data_ptr() if st is not None else None,
                                  sorted=int(bool(sorted)), lengths=_lengths_ptr(lengths, x, batch),
                                  share_threshold=int(bool(share_threshold))))
    if stats:
        return vals, idx, st
    return vals, idx


def topk_sample(x, k: int, B: int, B2: int, u, seed: int = 0, *, temperature: float = 1.0,
                top_p: float = 1.0, split: int = 0, waves: int = 0, kernel: int = 0, lengths=None,
                stream=None):
    """Top-k, softmax and one draw per row, fused into the output of the call.

    ``u``: a float32 device tensor of ``batch`` draws in [0, 1). Returns
    (vals, idx, probs, sampled): the k results of each row largest first, their
    softmax at ``temperature`` (float32), and the column drawn by inverse CDF
    from the smallest prefix whose probability reaches ``top_p`` (int32, -1
    for a row with no finite result). Needs k <= 1024.
    """
    import torch

    if x.dim() != 2 or x.stride(1) != 1 or not x.is_cuda:
        raise ValueError("x must be a 2-D device tensor with unit stride along the row")
    if x.dtype == torch.float32:
        dt = DS_F32
    elif x.dtype == torch.bfloat16:
        dt = DS_BF16
    else:
        raise ValueError(f"unsupported dtype {x.dtype}")
    batch, n = x.shape
    if (u.dtype != torch.float32 or u.device != x.device or u.dim() != 1 or u.shape[0] != batch
            or not u.is_contiguous()):
        raise ValueError("u must be a contiguous float32 tensor of batch entries on x's device")
    row_stride = x.stride(0) if batch > 1 else n
    vals = torch.empty((batch, k), dtype=x.dtype, device=x.device)
    idx = torch.empty((batch, k), dtype=torch.int32, device=x.device)
    probs = torch.empty((batch, k), dtype=torch.float32, device=x.device)
    sampled = torch.empty((batch,), dtype=torch.int32, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    with torch.cuda.device(x.device):
        _check(deepselect_topk_ex(x.data_ptr(), dt, batch, n, row_stride, k, B, B2, seed,
                                  vals.data_ptr(), idx.data_ptr(), stream, split=split, waves=waves,
                                  kernel=kernel, sorted=1, lengths=_lengths_ptr(lengths, x, batch),
                                  probs=probs.data_ptr(), temperature=temperature, top_p=top_p,
                                  sample_u=u.data_ptr(), sample_idx=sampled.data_ptr()))
    return vals, idx, probs, sampled
