"""MI355X (gfx950) row-wise softmax with the online normalizer.

Thin Python binding over the C ABI of ``libonline_softmax.so`` (declared in
``include/online_softmax.h``).  The functions here only marshal arguments:
they take torch tensors that live on the GPU, pass their device pointers,
sizes and the current HIP stream to the library, and raise on a non-zero
status.  Every step of the computation runs in the library's HIP kernels.
PyTorch supplies device memory and streams.

Entry points (same names as the C ABI):
  os_softmax_forward(x, out=None)              y = softmax(x) over the last dim
  os_softmax_forward_tuned(x, lanes_per_row, vecs_per_lane, grid_blocks=0, out=None)
  os_softmax_stats(x) -> (m, d)                per-row normaliser state
  os_softmax_forward_lse(x, out=None, write_y=True) -> (y, lse)   y and the per-row logsumexp
  os_softmax_forward_split(x, splits=None, out=None, workspace=None)   rows split over workgroups
  os_softmax_forward_workspace_bytes(rows, splits), os_forward_split_plan(rows, cols, dtype)
  os_softmax_forward_split_noalloc(x, splits=None, out=None)   the same, scratch inside the library
  os_softmax_topk(x, K, splits=None) -> (probs, idx)   fused softmax + top-K (fp32 or bf16 x)
  os_softmax_topk_ex(x, K, splits, workspace) -> (probs, idx)   the same with the dtype passed through
  os_softmax_topk_split(x, K, splits, workspace) -> (probs, idx)
  os_softmax_topk_workspace_bytes(rows, K, splits), os_topk_plan(rows, cols, K)
  safe_softmax_forward(x, out=None)            three-pass baseline
  naive_softmax_forward(x, out=None)           unshifted two-pass baseline (overflows past x = 88.7)
  os_topk_select(x, K) -> (vals, idx)          top-K of the entries alone (the unfused pipelines' TopK)
  os_device_copy(src, dst)                     plain copy (bandwidth reference)
  os_device_copy_rows(src, dst)                copy with the row-per-workgroup pattern (reference)
  os_bench_exp(out, workgroups, iters, chains) exponential-rate microbenchmark
  os_device_read(src, sink)                    plain read (read-only bandwidth reference)
  os_attention_forward(q, k, v, scale=None, causal=False, out=None, lse=True) -> (o, lse)
                                               attention forward on the online normalizer (bf16, d = 128)
  os_forward_plan(cols, dtype) -> (lanes_per_row, vecs_per_lane)
  os_last_error(), os_version()

There is no fallback: if the library is missing the import fails.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch  # loaded first: its HIP runtime is the one the library binds to

__all__ = [
    "OS_F32", "OS_BF16", "OS_TOPK_KMAX", "OnlineSoftmaxError", "LIB_PATH", "lib",
    "os_softmax_forward", "os_softmax_forward_tuned", "os_softmax_stats", "os_softmax_forward_lse", "os_softmax_topk",
    "safe_softmax_forward", "os_device_copy", "os_device_copy_rows", "os_forward_plan", "os_last_error", "os_version",
    "os_softmax_topk_split", "os_softmax_topk_workspace_bytes", "os_topk_plan", "os_softmax_topk_ex",
    "os_softmax_forward_split", "os_softmax_forward_workspace_bytes", "os_forward_split_plan",
    "os_softmax_forward_split_noalloc", "OS_STATIC_SCRATCH_BYTES", "naive_softmax_forward", "os_topk_select",
    "os_bench_exp", "os_device_read", "os_attention_forward",
]

OS_OK, OS_EINVAL, OS_EUNSUPPORTED, OS_ELAUNCH = 0, -1, -2, -3
OS_F32, OS_BF16 = 0, 1
OS_TOPK_KMAX = 32
OS_STATIC_SCRATCH_BYTES = 1 << 20

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libonline_softmax.so")


class OnlineSoftmaxError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


def _hip_runtimes_mapped() -> set[str]:
    found = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                path = line.rsplit(" ", 1)[-1].strip()
                if "libamdhip64.so" in os.path.basename(path):
                    found.add(os.path.realpath(path))
    except OSError:
        pass
    return found


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
            "(or python online_normalizer_amd/build.py); there is no fallback")
    L = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError(f"two HIP runtimes are loaded in this process: {sorted(runtimes)}")
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sig = {
        "os_softmax_forward": [vp, vp, i64, i64, i32, vp],
        "os_softmax_forward_tuned": [vp, vp, i64, i64, i32, i32, i32, i32, vp],
        "os_forward_plan": [i64, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)],
        "os_softmax_stats": [vp, vp, vp, i64, i64, i32, vp],
        "os_softmax_forward_lse": [vp, vp, vp, i64, i64, i32, vp],
        "os_softmax_forward_split": [vp, vp, i64, i64, i32, i32, vp, i64, vp],
        "os_softmax_forward_split_noalloc": [vp, vp, i64, i64, i32, i32, vp],
        "os_forward_split_plan": [i64, i64, i32],
        "os_softmax_topk": [vp, vp, vp, i64, i64, i32, vp],
        "safe_softmax_forward": [vp, vp, i64, i64, i32, vp],
        "naive_softmax_forward": [vp, vp, i64, i64, i32, vp],
        "os_topk_select": [vp, i32, vp, vp, i64, i64, i32, vp],
        "os_device_copy": [vp, vp, i64, vp],
        "os_device_copy_rows": [vp, vp, i64, i64, vp],
        "os_bench_exp": [vp, i64, i32, i32, vp],
        "os_device_read": [vp, i64, vp, i64, vp],
        "os_attention_forward": [vp, vp, vp, vp, vp, i64, i64, i64, i32, ctypes.c_float, i32, vp],
        "os_version": [],
        "os_softmax_topk_split": [vp, vp, vp, i64, i64, i32, i32, vp, i64, vp],
        "os_topk_plan": [i64, i64, i32],
        "os_softmax_topk_ex": [vp, i32, vp, vp, i64, i64, i32, i32, vp, i64, vp],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = i32
    L.os_softmax_topk_workspace_bytes.argtypes = [i64, i32, i32]
    L.os_softmax_topk_workspace_bytes.restype = i64
    L.os_softmax_forward_workspace_bytes.argtypes = [i64, i32]
    L.os_softmax_forward_workspace_bytes.restype = i64
    L.os_last_error.argtypes = []
    L.os_last_error.restype = ctypes.c_char_p
    return L


_LIB: ctypes.CDLL | None = None


def lib() -> ctypes.CDLL:
    """The loaded C library (raw ctypes handle)."""
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


lib()


def os_last_error() -> str:
    return lib().os_last_error().decode()


def os_version() -> int:
    return lib().os_version()


def _check(fn: str, status: int):
    if status != OS_OK:
        raise OnlineSoftmaxError(fn, status, os_last_error())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return OS_F32
    if t.dtype == torch.bfloat16:
        return OS_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _rows_cols(x: torch.Tensor):
    if x.dim() == 0:
        raise ValueError("softmax needs at least one dimension")
    if not x.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not x.is_contiguous():
        raise ValueError("tensors must be contiguous (row stride == cols)")
    cols = x.shape[-1]
    rows = math.prod(x.shape[:-1])
    return rows, cols


def _stream(x: torch.Tensor) -> int:
    return torch.cuda.current_stream(x.device).cuda_stream


def _out_like(x, out):
    if out is None:
        return torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype or out.device != x.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor with the input's shape, dtype and device")
    return out


def _whole(t: torch.Tensor, what: str, like: torch.Tensor | None = None):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous GPU tensor")
    if like is not None and t.device != like.device:
        raise ValueError(f"{what} must be on the input's device")


def os_softmax_forward(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    rows, cols = _rows_cols(x)
    out = _out_like(x, out)
    _check("os_softmax_forward",
           lib().os_softmax_forward(x.data_ptr(), out.data_ptr(), rows, cols, _dtype_code(x), _stream(x)))
    return out


def os_softmax_forward_tuned(x: torch.Tensor, lanes_per_row: int, vecs_per_lane: int,
                             grid_blocks: int = 0, out: torch.Tensor | None = None) -> torch.Tensor:
    rows, cols = _rows_cols(x)
    out = _out_like(x, out)
    _check("os_softmax_forward_tuned",
           lib().os_softmax_forward_tuned(x.data_ptr(), out.data_ptr(), rows, cols, _dtype_code(x),
                                          lanes_per_row, vecs_per_lane, grid_blocks, _stream(x)))
    return out


def os_forward_plan(cols: int, dtype: torch.dtype = torch.float32) -> tuple[int, int]:
    code = OS_BF16 if dtype == torch.bfloat16 else OS_F32
    a, b = ctypes.c_int(), ctypes.c_int()
    _check("os_forward_plan", lib().os_forward_plan(cols, code, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def os_softmax_stats(x: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    rows, cols = _rows_cols(x)
    shape = x.shape[:-1]
    m = torch.empty(shape, dtype=torch.float32, device=x.device)
    d = torch.empty(shape, dtype=torch.float32, device=x.device)
    _check("os_softmax_stats",
           lib().os_softmax_stats(x.data_ptr(), m.data_ptr(), d.data_ptr(), rows, cols, _dtype_code(x),
                                  _stream(x)))
    return m, d


def os_softmax_forward_lse(x: torch.Tensor, out: torch.Tensor | None = None,
                           write_y: bool = True) -> tuple[torch.Tensor | None, torch.Tensor]:
    """y = softmax(x) and L = logsumexp(x) over the last dim in one launch;
    with write_y=False only L is computed (y is None)."""
    rows, cols = _rows_cols(x)
    y = _out_like(x, out) if write_y else None
    lse = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _check("os_softmax_forward_lse",
           lib().os_softmax_forward_lse(x.data_ptr(), None if y is None else y.data_ptr(), lse.data_ptr(), rows,
                                        cols, _dtype_code(x), _stream(x)))
    return y, lse


def os_topk_plan(rows: int, cols: int, K: int) -> int:
    return lib().os_topk_plan(rows, cols, K)


def os_softmax_topk_workspace_bytes(rows: int, K: int, splits: int) -> int:
    n = lib().os_softmax_topk_workspace_bytes(rows, K, splits)
    if n < 0:
        raise OnlineSoftmaxError("os_softmax_topk_workspace_bytes", n, os_last_error())
    return n


# Workspaces of the split launches (top-K and forward), one per (device,
# stream): calls on one stream run in order, so they can share it.
_SPLIT_WS: dict[tuple[int, int], torch.Tensor] = {}


def _split_workspace(x: torch.Tensor, nbytes: int) -> torch.Tensor:
    key = (x.device.index, _stream(x))
    ws = _SPLIT_WS.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=x.device)
        _SPLIT_WS[key] = ws
    return ws


def _topk_out(x, K, probs=None, idx=None):
    """rows, cols and the (probs or values, indices) outputs: new tensors, or
    the caller's, checked to be contiguous [..., K] float32 / int32 tensors on
    x's device (the library writes rows * K entries through their pointers)."""
    rows, cols = _rows_cols(x)
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("top-K takes float32 or bfloat16 input")
    shape = (*x.shape[:-1], K)
    for name, t, dt in (("probs", probs, torch.float32), ("idx", idx, torch.int32)):
        if t is not None and (tuple(t.shape) != shape or t.dtype != dt or t.device != x.device
                              or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous {dt} tensor of shape {shape} on {x.device}")
    probs = torch.empty(shape, dtype=torch.float32, device=x.device) if probs is None else probs
    idx = torch.empty(shape, dtype=torch.int32, device=x.device) if idx is None else idx
    return rows, cols, probs, idx


def os_softmax_topk_split(x: torch.Tensor, K: int, splits: int,
                          workspace: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    rows, cols, probs, idx = _topk_out(x, K)
    _whole(workspace, "workspace", x)
    _check("os_softmax_topk_split",
           lib().os_softmax_topk_split(x.data_ptr(), probs.data_ptr(), idx.data_ptr(), rows, cols, K, splits,
                                       workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                       _stream(x)))
    return probs, idx


def os_softmax_topk(x: torch.Tensor, K: int, splits: int | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Fused softmax + top-K.  splits=None asks the library's plan; a split
    launch uses a workspace cached per (device, stream)."""
    rows, cols, probs, idx = _topk_out(x, K)
    if splits is None:
        splits = os_topk_plan(rows, cols, K)
    if x.dtype == torch.bfloat16:
        ws = _split_workspace(x, os_softmax_topk_workspace_bytes(rows, K, splits))
        return os_softmax_topk_ex(x, K, splits, ws, probs, idx)
    if splits == 1:
        _check("os_softmax_topk",
               lib().os_softmax_topk(x.data_ptr(), probs.data_ptr(), idx.data_ptr(), rows, cols, K, _stream(x)))
        return probs, idx
    ws = _split_workspace(x, os_softmax_topk_workspace_bytes(rows, K, splits))
    return os_softmax_topk_split(x, K, splits, ws)


def os_device_copy_rows(src: torch.Tensor, dst: torch.Tensor) -> torch.Tensor:
    """Copy src (rows x row_bytes, row_bytes <= 128 KiB) with the register-resident
    forward's access pattern (a bandwidth reference)."""
    rows, cols = _rows_cols(src)
    if dst.shape != src.shape or dst.dtype != src.dtype or not dst.is_contiguous() or dst.device != src.device:
        raise ValueError("dst must be a contiguous tensor like src, on its device")
    _check("os_device_copy_rows", lib().os_device_copy_rows(src.data_ptr(), dst.data_ptr(), rows,
                                                            cols * src.element_size(), _stream(src)))
    return dst


def os_forward_split_plan(rows: int, cols: int, dtype: torch.dtype = torch.float32) -> int:
    return lib().os_forward_split_plan(rows, cols, OS_BF16 if dtype == torch.bfloat16 else OS_F32)


def os_softmax_forward_workspace_bytes(rows: int, splits: int) -> int:
    n = lib().os_softmax_forward_workspace_bytes(rows, splits)
    if n < 0:
        raise OnlineSoftmaxError("os_softmax_forward_workspace_bytes", n, os_last_error())
    return n


def os_softmax_forward_split(x: torch.Tensor, splits: int | None = None, out: torch.Tensor | None = None,
                             workspace: torch.Tensor | None = None) -> torch.Tensor:
    """The forward with each row split over several workgroups.  splits=None
    asks the library's plan; without a workspace one cached per (device,
    stream) is used."""
    rows, cols = _rows_cols(x)
    out = _out_like(x, out)
    if splits is None:
        splits = os_forward_split_plan(rows, cols, x.dtype)
    if workspace is None:
        workspace = _split_workspace(x, os_softmax_forward_workspace_bytes(rows, splits))
    _whole(workspace, "workspace", x)
    _check("os_softmax_forward_split",
           lib().os_softmax_forward_split(x.data_ptr(), out.data_ptr(), rows, cols, _dtype_code(x), splits,
                                          workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                          _stream(x)))
    return out


def os_softmax_forward_split_noalloc(x: torch.Tensor, splits: int | None = None,
                                     out: torch.Tensor | None = None) -> torch.Tensor:
    """The split forward on the library's own device-resident scratch (no
    workspace, no allocation inside the call; pass `out` to allocate nothing
    here either).  splits=None asks the library's plan."""
    rows, cols = _rows_cols(x)
    out = _out_like(x, out)
    if splits is None:
        splits = os_forward_split_plan(rows, cols, x.dtype)
    _check("os_softmax_forward_split_noalloc",
           lib().os_softmax_forward_split_noalloc(x.data_ptr(), out.data_ptr(), rows, cols, _dtype_code(x), splits,
                                                  _stream(x)))
    return out


def os_softmax_topk_ex(x: torch.Tensor, K: int, splits: int, workspace: torch.Tensor | None,
                       probs: torch.Tensor | None = None,
                       idx: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Fused softmax + top-K for float32 or bfloat16 input (dtype from the tensor).
    workspace may be None when splits == 1."""
    rows, cols, probs, idx = _topk_out(x, K, probs, idx)
    if workspace is not None:
        _whole(workspace, "workspace", x)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("os_softmax_topk_ex",
           lib().os_softmax_topk_ex(x.data_ptr(), _dtype_code(x), probs.data_ptr(), idx.data_ptr(), rows, cols, K,
                                    splits, ws_ptr, ws_bytes, _stream(x)))
    return probs, idx


def safe_softmax_forward(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    rows, cols = _rows_cols(x)
    out = _out_like(x, out)
    _check("safe_softmax_forward",
           lib().safe_softmax_forward(x.data_ptr(), out.data_ptr(), rows, cols, _dtype_code(x), _stream(x)))
    return out


def naive_softmax_forward(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    rows, cols = _rows_cols(x)
    out = _out_like(x, out)
    _check("naive_softmax_forward",
           lib().naive_softmax_forward(x.data_ptr(), out.data_ptr(), rows, cols, _dtype_code(x), _stream(x)))
    return out


def os_topk_select(x: torch.Tensor, K: int, vals: torch.Tensor | None = None,
                   idx: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """The K largest entries of each row (value desc, index asc) and their columns."""
    rows, cols, vals, idx = _topk_out(x, K, vals, idx)
    _check("os_topk_select",
           lib().os_topk_select(x.data_ptr(), _dtype_code(x), vals.data_ptr(), idx.data_ptr(), rows, cols, K,
                                _stream(x)))
    return vals, idx


def os_bench_exp(out: torch.Tensor, workgroups: int, iters: int, chains: int) -> torch.Tensor:
    """Launch the exponential-rate microbenchmark (workgroups * 256 * iters *
    chains exponentials); out: float32 with at least workgroups * 256 elements."""
    if out.dtype != torch.float32 or not out.is_cuda or not out.is_contiguous() or out.numel() < workgroups * 256:
        raise ValueError("out must be a float32 GPU tensor of at least workgroups * 256 elements")
    _check("os_bench_exp", lib().os_bench_exp(out.data_ptr(), workgroups, iters, chains, _stream(out)))
    return out


def os_device_read(src: torch.Tensor, sink: torch.Tensor) -> torch.Tensor:
    """Read all of src (a plain read, the read-only bandwidth reference); sink:
    float32, at least 4 * min(2048, ceil(bytes / 4096)) elements."""
    if sink.dtype != torch.float32 or not sink.is_cuda or not sink.is_contiguous() or sink.device != src.device:
        raise ValueError("sink must be a contiguous float32 tensor on src's device")
    _whole(src, "src")
    nbytes = src.numel() * src.element_size()
    _check("os_device_read", lib().os_device_read(src.data_ptr(), nbytes, sink.data_ptr(), sink.numel(), _stream(src)))
    return sink


def os_attention_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
                         causal: bool = False, out: torch.Tensor | None = None,
                         lse: bool = True) -> tuple[torch.Tensor, torch.Tensor | None]:
    """O = softmax(scale Q K^T) V per head for bf16 q [..., nq, d], k and v
    [..., nk, d] (contiguous; the leading dimensions are the heads), and the
    per-row logsumexp (float32 [..., nq]) when lse is true.  scale defaults to
    1/sqrt(d)."""
    for t in (q, k, v):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.dim() < 2:
            raise TypeError("q, k, v must be contiguous bfloat16 GPU tensors [..., n, d]")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on one device")
    d = q.shape[-1]
    if k.shape != v.shape or k.shape[:-2] != q.shape[:-2] or k.shape[-1] != d:
        raise ValueError("k and v must be [..., nk, d] with q's leading dimensions and d")
    heads = q.numel() // max(1, q.shape[-2] * d) if q.shape[-2] * d else 0
    nq, nk = q.shape[-2], k.shape[-2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _out_like(q, out)
    L = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device) if lse else None
    _check("os_attention_forward",
           lib().os_attention_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                      None if L is None else L.data_ptr(), heads, nq, nk, d, float(scale),
                                      int(bool(causal)), _stream(q)))
    return out, L


def os_device_copy(src: torch.Tensor, dst: torch.Tensor) -> torch.Tensor:
    _whole(src, "src")
    _whole(dst, "dst", src)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst is smaller than src")
    _check("os_device_copy", lib().os_device_copy(src.data_ptr(), dst.data_ptr(), nbytes, _stream(src)))
    return dst
