"""Python binding of libawq_mi355x.so, the MI355X (gfx950) W4A16 library.

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream. The binding raises
if the library has not been built or a tensor is not a GPU tensor; there is
no CPU fallback.

Entry points (same names as the C ABI in include/awq.h):
    awq_quantize(w, group_size=128, channel_scale=None)  -> qweight, scales, zeros
    awq_gemm(x, qweight, scales, zeros, group_size=128, path=0, workspace=None) -> y
        (awq_gemm_ex when a workspace from gemm_workspace(M, N, K) is given)
    awq_activation_absmean(x) -> m
    awq_scale_search(w, x, group_size=128, alphas=None) -> losses, best_index, best_scales
"""

from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libawq_mi355x.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "awq.h")

AWQ_OK = 0
STATUS_NAMES = {
    0: "AWQ_OK", 1: "AWQ_ERR_NULL", 2: "AWQ_ERR_SHAPE", 3: "AWQ_ERR_ALIGN",
    4: "AWQ_ERR_CONFIG", 5: "AWQ_ERR_WORKSPACE", 6: "AWQ_ERR_HIP",
}
PATH_AUTO, PATH_GEMV, PATH_GEMM, PATH_SKINNY, PATH_COLTILE = 0, 1, 2, 3, 4
QUANT_ASYMMETRIC, QUANT_SYMMETRIC = 0, 1

_lib = None


class AwqError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed: {message}")
        self.status = status


def lib_path() -> str:
    return LIB_PATH


def load() -> ctypes.CDLL:
    """Loads the built library (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m weight_only_int4_quantize_amd.build` "
            "(there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    c_i64, c_int, c_vp, c_sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    L.awq_status_string.restype = ctypes.c_char_p
    L.awq_status_string.argtypes = [c_int]
    L.awq_version.restype = c_int
    L.awq_version.argtypes = []
    L.awq_quantize.restype = c_int
    L.awq_quantize.argtypes = [c_vp, c_vp, c_i64, c_i64, c_int, c_vp, c_vp, c_vp, c_vp]
    L.awq_quantize_ex.restype = c_int
    L.awq_quantize_ex.argtypes = [c_vp, c_vp, c_i64, c_i64, c_int, c_int, ctypes.c_double, c_vp, c_vp, c_vp, c_vp]
    L.awq_clip_search_workspace_bytes.restype = c_sz
    L.awq_clip_search_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, c_int, c_int, c_int]
    L.awq_clip_search.restype = c_int
    L.awq_clip_search.argtypes = [c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_int, c_int, c_vp, c_int, c_vp, c_sz,
                                  c_vp, c_vp, c_vp]
    L.awq_gemm.restype = c_int
    L.awq_gemm.argtypes = [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_int, c_vp, c_vp]
    L.awq_gemm_path.restype = c_int
    L.awq_gemm_path.argtypes = [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_int, c_vp, c_int, c_vp]
    L.awq_gemm_workspace_bytes.restype = c_sz
    L.awq_gemm_workspace_bytes.argtypes = [c_i64, c_i64, c_i64]
    L.awq_gemm_ex.restype = c_int
    L.awq_gemm_ex.argtypes = [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_int, c_vp, c_int, c_vp, c_sz, c_vp]
    L.awq_gemm_kernel.restype = c_int
    L.awq_gemm_kernel.argtypes = [c_i64, c_i64, c_i64, c_int, c_int, c_int]
    L.awq_gemm_noalloc.restype = c_int
    L.awq_gemm_noalloc.argtypes = [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_int, c_vp, c_int, c_vp]
    L.awq_gemm_grouped.restype = c_int
    L.awq_gemm_grouped.argtypes = [c_vp, c_int, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_int, c_vp, c_vp]
    L.awq_activation_absmean_workspace_bytes.restype = c_sz
    L.awq_activation_absmean_workspace_bytes.argtypes = [c_i64, c_i64]
    L.awq_activation_absmean.restype = c_int
    L.awq_activation_absmean.argtypes = [c_vp, c_i64, c_i64, c_vp, c_vp, c_sz, c_vp]
    L.awq_scale_search_workspace_bytes.restype = c_sz
    L.awq_scale_search_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, c_int, c_int]
    L.awq_scale_search.restype = c_int
    L.awq_scale_search.argtypes = [c_vp, c_vp, c_i64, c_i64, c_i64, c_int, c_vp, c_int, c_vp, c_sz,
                                   c_vp, c_vp, c_vp, c_vp]
    L.awq_select_salient.restype = c_int
    L.awq_select_salient.argtypes = [c_vp, c_i64, c_int, c_vp, c_vp]
    L.awq_quantize_salient.restype = c_int
    L.awq_quantize_salient.argtypes = [c_vp, c_i64, c_i64, c_int, c_int, c_vp, c_int, c_vp, c_vp, c_vp, c_vp, c_vp]
    L.awq_salient_apply.restype = c_int
    L.awq_salient_apply.argtypes = [c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_int, c_vp, c_vp]
    L.awq_salient_count.restype = c_i64
    L.awq_salient_count.argtypes = [c_i64]
    L.awq_salient_loss_workspace_bytes.restype = c_sz
    L.awq_salient_loss_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, c_int, c_int]
    L.awq_salient_loss.restype = c_int
    L.awq_salient_loss.argtypes = [c_vp, c_vp, c_i64, c_i64, c_i64, c_int, c_int, c_int, c_vp, c_sz, c_vp, c_vp,
                                   c_vp, c_vp]
    L.awq_quantize_w8.restype = c_int
    L.awq_quantize_w8.argtypes = [c_vp, c_vp, c_i64, c_i64, c_int, c_int, c_vp, c_vp, c_vp, c_vp]
    L.awq_gemm_w8.restype = c_int
    L.awq_gemm_w8.argtypes = [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_int, c_vp, c_int, c_vp, c_sz, c_vp]
    _lib = L
    return L


def header_functions() -> list:
    """Names of the functions include/awq.h declares."""
    with open(HEADER, encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(awq_[a-z0-9_]+)\s*\(", text)))


def _check(fn: str, status: int) -> None:
    if status != AWQ_OK:
        msg = load().awq_status_string(status).decode()
        raise AwqError(fn, status, msg)


def _torch():
    import torch
    return torch


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _need_gpu(name: str, t, dtype=None) -> None:
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_out(qweight, scales, zeros, q_shape, sz_shape, device) -> None:
    """Caller-given quantize outputs: int32 qweight and fp16 scales / zeros of
    exactly the shapes the call writes, contiguous, on the input's device."""
    torch = _torch()
    for name, t, dtype, shape in (("qweight", qweight, torch.int32, q_shape), ("scales", scales, torch.float16, sz_shape),
                                  ("zeros", zeros, torch.float16, sz_shape)):
        _need_gpu(name, t, dtype)
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must be {list(shape)}, got {list(t.shape)}")
        if t.device != device:
            raise ValueError(f"{name} must be on {device}")


def awq_quantize(w, group_size: int = 128, channel_scale=None, out=None, symmetric: bool = False,
                 clip_fraction: float = 0.0):
    """Group-wise INT4 quantization of w[N, K] (fp16), asymmetric by default
    (awq_quantize); symmetric=True or clip_fraction > 0 go to
    awq_quantize_ex (symmetric map; percentile clip of each group).

    Returns (qweight int32 [N, K/8] holding the uint32 words, scales fp16
    [N, K/G], zeros fp16 [N, K/G]). channel_scale: optional fp32 [K]."""
    torch = _torch()
    _need_gpu("w", w, torch.float16)
    if w.dim() != 2:
        raise ValueError("w must be 2-D [N, K]")
    N, K = w.shape
    if channel_scale is not None:
        _need_gpu("channel_scale", channel_scale, torch.float32)
        if channel_scale.numel() != K:
            raise ValueError("channel_scale must have K elements")
    ng = K // group_size if group_size > 0 else 0
    if out is None:
        dev = w.device
        qweight = torch.empty((N, max(K // 8, 0)), dtype=torch.int32, device=dev)
        scales = torch.empty((N, ng), dtype=torch.float16, device=dev)
        zeros = torch.empty((N, ng), dtype=torch.float16, device=dev)
    else:
        qweight, scales, zeros = out
        _need_out(qweight, scales, zeros, (N, K // 8), (N, ng), w.device)
    if symmetric or clip_fraction != 0.0:
        mode = QUANT_SYMMETRIC if symmetric else QUANT_ASYMMETRIC
        st = load().awq_quantize_ex(_ptr(w), _ptr(channel_scale), N, K, group_size, mode, float(clip_fraction),
                                    _ptr(qweight), _ptr(scales), _ptr(zeros), _stream(w.device))
        _check("awq_quantize_ex", st)
    else:
        st = load().awq_quantize(_ptr(w), _ptr(channel_scale), N, K, group_size, _ptr(qweight),
                                 _ptr(scales), _ptr(zeros), _stream(w.device))
        _check("awq_quantize", st)
    return qweight, scales, zeros


KERNEL_NAMES = {1: "gemv", 2: "gemm", 3: "skinny", 4: "coltile"}


def gemm_kernel(M: int, N: int, K: int, group_size: int = 128, path: int = PATH_AUTO,
                workspace: bool = False) -> str:
    """Name of the kernel awq_gemm runs for this shape (awq_gemm_kernel)."""
    k = int(load().awq_gemm_kernel(M, N, K, group_size, path, int(workspace)))
    if k < 0:
        raise AwqError("awq_gemm_kernel", 4, "the path cannot take this shape")
    return KERNEL_NAMES[k]


def gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(load().awq_gemm_workspace_bytes(M, N, K))


def gemm_workspace(M: int, N: int, K: int, device=None):
    """A zero-filled uint8 GPU tensor of awq_gemm_workspace_bytes(M, N, K)
    bytes: awq_gemm_ex's workspace for this shape and for any other whose
    awq_gemm_workspace_bytes is no larger (today the size depends on M
    only). Each call leaves it ready for the next, without clearing."""
    torch = _torch()
    nbytes = gemm_workspace_bytes(M, N, K)
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device or "cuda")


def awq_gemm(x, qweight, scales, zeros, group_size: int = 128, path: int = PATH_AUTO, out=None,
             workspace=None):
    """y[M, N] = x[M, K] . dequant(Wq)^T in fp16 (fp32 accumulation).

    With a workspace (see gemm_workspace) the call goes to awq_gemm_ex,
    which may split output tiles' K loops across blocks (stream-K)."""
    torch = _torch()
    _need_gpu("x", x, torch.float16)
    _need_gpu("qweight", qweight, torch.int32)
    _need_gpu("scales", scales, torch.float16)
    _need_gpu("zeros", zeros, torch.float16)
    if x.dim() != 2 or qweight.dim() != 2:
        raise ValueError("x and qweight must be 2-D")
    M, K = x.shape
    N = qweight.shape[0]
    if qweight.shape[1] * 8 != K:
        raise ValueError(f"qweight has {qweight.shape[1]} words per row, K={K} needs {K // 8}")
    if scales.shape != (N, K // group_size) or zeros.shape != scales.shape:
        raise ValueError("scales/zeros must be [N, K/group_size]")
    y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=x.device)
    if out is not None:
        _need_gpu("out", y, torch.float16)
        if tuple(y.shape) != (M, N):
            raise ValueError("out must be [M, N]")
    if workspace is None:
        st = load().awq_gemm_path(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(zeros), M, N, K, group_size,
                                  _ptr(y), int(path), _stream(x.device))
        _check("awq_gemm", st)
    else:
        _need_gpu("workspace", workspace, torch.uint8)
        st = load().awq_gemm_ex(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(zeros), M, N, K, group_size,
                                _ptr(y), int(path), _ptr(workspace), workspace.numel(), _stream(x.device))
        _check("awq_gemm_ex", st)
    return y


def awq_gemm_noalloc(x, qweight, scales, zeros, group_size: int = 128, path: int = PATH_AUTO, out=None):
    """awq_gemm_noalloc: awq_gemm with the skinny kernel's K-split scratch
    held by the library (no workspace, no device allocation in the call;
    calls on one device must not overlap). Pass `out` to keep the binding
    from allocating y."""
    torch = _torch()
    _need_gpu("x", x, torch.float16)
    _need_gpu("qweight", qweight, torch.int32)
    _need_gpu("scales", scales, torch.float16)
    _need_gpu("zeros", zeros, torch.float16)
    M, K = x.shape
    N = qweight.shape[0]
    if qweight.shape != (N, K // 8) or K % 8:
        raise ValueError(f"qweight must be [N, K/8] = [{N}, {K // 8}]")
    if scales.shape != (N, K // group_size) or zeros.shape != scales.shape:
        raise ValueError("scales/zeros must be [N, K/group_size]")
    y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=x.device)
    _need_gpu("out", y, torch.float16)
    if tuple(y.shape) != (M, N):
        raise ValueError("out must be [M, N]")
    st = load().awq_gemm_noalloc(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(zeros), M, N, K, group_size, _ptr(y),
                                 int(path), _stream(x.device))
    _check("awq_gemm_noalloc", st)
    return y


def awq_gemm_grouped(x, layers, group_size: int = 128, outs=None):
    """y_i = x . dequant(Wq_i)^T for layers [(qweight, scales, zeros), ...]
    (1 to 4) that share x: one GEMV or column-tile launch over their
    stacked rows where awq_gemm would take that kernel, else one awq_gemm
    per layer. Returns the list of y_i (`outs`, when given, receives them)."""
    torch = _torch()
    _need_gpu("x", x, torch.float16)
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    M, K = x.shape
    n = len(layers)
    ys = list(outs) if outs is not None else [None] * n
    if len(ys) != n:
        raise ValueError("outs must hold one tensor per layer")
    Ns = []
    for i, (qw, sc, zr) in enumerate(layers):
        _need_gpu("qweight", qw, torch.int32)
        _need_gpu("scales", sc, torch.float16)
        _need_gpu("zeros", zr, torch.float16)
        N = qw.shape[0]
        if qw.dim() != 2 or qw.shape[1] * 8 != K:
            raise ValueError(f"layer {i}: qweight must be [N, K/8] with K = {K}")
        if sc.shape != (N, K // group_size) or zr.shape != sc.shape:
            raise ValueError(f"layer {i}: scales/zeros must be [N, K/group_size]")
        if ys[i] is None:
            ys[i] = torch.empty((M, N), dtype=torch.float16, device=x.device)
        _need_gpu("out", ys[i], torch.float16)
        if tuple(ys[i].shape) != (M, N):
            raise ValueError(f"layer {i}: out must be [M, N]")
        Ns.append(N)
    arr = ctypes.c_void_p * max(n, 1)
    st = load().awq_gemm_grouped(
        _ptr(x), n, arr(*[_ptr(l[0]) for l in layers]), arr(*[_ptr(l[1]) for l in layers]),
        arr(*[_ptr(l[2]) for l in layers]), (ctypes.c_int64 * max(n, 1))(*Ns), M, K, group_size,
        arr(*[_ptr(y) for y in ys]), _stream(x.device))
    _check("awq_gemm_grouped", st)
    return ys


def awq_activation_absmean(x):
    """m[k] = max(mean_t |x[t, k]|, 1e-8) in fp64, x fp16 [T, K]."""
    torch = _torch()
    _need_gpu("x", x, torch.float16)
    T, K = x.shape
    L = load()
    m = torch.empty(K, dtype=torch.float64, device=x.device)
    nbytes = L.awq_activation_absmean_workspace_bytes(T, K)
    ws = torch.empty(max(nbytes, 8), dtype=torch.uint8, device=x.device)
    st = L.awq_activation_absmean(_ptr(x), T, K, _ptr(m), _ptr(ws), nbytes, _stream(x.device))
    _check("awq_activation_absmean", st)
    return m


def scale_search_workspace_bytes(N: int, K: int, T: int, group_size: int = 128, n_alpha: int = 20) -> int:
    return int(load().awq_scale_search_workspace_bytes(N, K, T, group_size, n_alpha))


def awq_scale_search(w, x, group_size: int = 128, alphas=None, workspace=None, n_alpha: int = 20):
    """AWQ scale search over an alpha grid.

    Returns (losses: numpy float64 [n_alpha], best_index: int,
    best_scales: fp32 GPU tensor [K])."""
    import numpy as np
    torch = _torch()
    _need_gpu("w", w, torch.float16)
    _need_gpu("x", x, torch.float16)
    N, K = w.shape
    T = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("x must be [T, K] with the K of w")
    # no grid given: the library's default grid of n_alpha points
    if alphas is not None:
        alphas = np.ascontiguousarray(alphas, dtype=np.float64)
    n_alpha = int(alphas.size) if alphas is not None else int(n_alpha)
    L = load()
    nbytes = L.awq_scale_search_workspace_bytes(N, K, T, group_size, n_alpha)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=w.device)
    losses = np.zeros(n_alpha, dtype=np.float64)
    best = ctypes.c_int(-1)
    best_scales = torch.empty(K, dtype=torch.float32, device=w.device)
    st = L.awq_scale_search(_ptr(w), _ptr(x), N, K, T, group_size,
                            None if alphas is None else alphas.ctypes.data_as(ctypes.c_void_p), n_alpha,
                            _ptr(workspace), workspace.numel(),
                            losses.ctypes.data_as(ctypes.c_void_p), ctypes.addressof(best),
                            _ptr(best_scales), _stream(w.device))
    _check("awq_scale_search", st)
    return losses, int(best.value), best_scales


def awq_clip_search(w, x, fractions, group_size: int = 128, channel_scale=None, symmetric: bool = False,
                    workspace=None):
    """Clip-fraction search (awq_clip_search). Returns (losses: numpy float64
    [n], best_index: int)."""
    import numpy as np
    torch = _torch()
    _need_gpu("w", w, torch.float16)
    _need_gpu("x", x, torch.float16)
    N, K = w.shape
    T = x.shape[0]
    if channel_scale is not None:
        _need_gpu("channel_scale", channel_scale, torch.float32)
        if channel_scale.numel() != K:
            raise ValueError("channel_scale must have K elements")
    fr = np.ascontiguousarray(fractions, dtype=np.float64)
    n = int(fr.size)
    L = load()
    nbytes = L.awq_clip_search_workspace_bytes(N, K, T, group_size, n, int(channel_scale is not None))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=w.device)
    losses = np.zeros(n, dtype=np.float64)
    best = ctypes.c_int(-1)
    mode = QUANT_SYMMETRIC if symmetric else QUANT_ASYMMETRIC
    st = L.awq_clip_search(_ptr(w), _ptr(x), _ptr(channel_scale), N, K, T, group_size, mode,
                           fr.ctypes.data_as(ctypes.c_void_p), n, _ptr(workspace), workspace.numel(),
                           losses.ctypes.data_as(ctypes.c_void_p), ctypes.addressof(best), _stream(w.device))
    _check("awq_clip_search", st)
    return losses, int(best.value)


# ---------------------------------------------------------------- mixed precision (fp16 salient channels)

def select_salient(m, n_salient: int):
    """awq_select_salient: int32 [n_salient] channel indices, largest m first
    (m: fp64 GPU tensor [K], e.g. awq_activation_absmean's)."""
    torch = _torch()
    _need_gpu("m", m, torch.float64)
    idx = torch.empty(max(n_salient, 1), dtype=torch.int32, device=m.device)[:n_salient]
    _check("awq_select_salient", load().awq_select_salient(_ptr(m), m.numel(), n_salient, _ptr(idx),
                                                           _stream(m.device)))
    return idx


def awq_quantize_salient(w, group_size: int, idx, symmetric: bool = False):
    """awq_quantize_salient: (qweight, scales, zeros, w_salient fp16
    [n_salient, N]) for the channels idx (int32 GPU tensor)."""
    torch = _torch()
    _need_gpu("w", w, torch.float16)
    _need_gpu("idx", idx, torch.int32)
    N, K = w.shape
    n = idx.numel()
    dev = w.device
    qweight = torch.empty((N, max(K // 8, 0)), dtype=torch.int32, device=dev)
    ng = K // group_size if group_size > 0 else 0
    scales = torch.empty((N, ng), dtype=torch.float16, device=dev)
    zeros = torch.empty((N, ng), dtype=torch.float16, device=dev)
    w_sal = torch.empty((n, N), dtype=torch.float16, device=dev)
    mode = QUANT_SYMMETRIC if symmetric else QUANT_ASYMMETRIC
    st = load().awq_quantize_salient(_ptr(w), N, K, group_size, mode, _ptr(idx), n, _ptr(qweight), _ptr(scales),
                                     _ptr(zeros), _ptr(w_sal), _stream(dev))
    _check("awq_quantize_salient", st)
    return qweight, scales, zeros, w_sal


def awq_salient_apply(x, idx, w_salient, y):
    """awq_salient_apply: y (fp16 [M, N]) += x[:, idx] . w_salient, in place."""
    torch = _torch()
    _need_gpu("x", x, torch.float16)
    _need_gpu("idx", idx, torch.int32)
    _need_gpu("w_salient", w_salient, torch.float16)
    _need_gpu("y", y, torch.float16)
    M, K = x.shape
    n, N = w_salient.shape
    if idx.numel() != n or y.shape != (M, N):
        raise ValueError("shapes: idx [n], w_salient [n, N], y [M, N]")
    _check("awq_salient_apply", load().awq_salient_apply(_ptr(x), _ptr(idx), _ptr(w_salient), M, N, K, n, _ptr(y),
                                                         _stream(x.device)))
    return y


def awq_gemm_salient(x, qweight, scales, zeros, idx, w_salient, group_size: int = 128, path: int = PATH_AUTO,
                     out=None, workspace=None):
    """The mixed layer: awq_gemm then awq_salient_apply on the same stream."""
    y = awq_gemm(x, qweight, scales, zeros, group_size, path=path, out=out, workspace=workspace)
    return awq_salient_apply(x, idx, w_salient, y)


def awq_salient_loss(w, x, group_size: int = 128, n_salient: int | None = None, symmetric: bool = False,
                     workspace=None):
    """awq_salient_loss: (loss_rtn, loss_salient, idx int32 GPU tensor).
    n_salient defaults to the library's awq_salient_count(K), the pages' 1 %."""
    import numpy as np
    torch = _torch()
    _need_gpu("w", w, torch.float16)
    _need_gpu("x", x, torch.float16)
    N, K = w.shape
    T = x.shape[0]
    L = load()
    n = int(L.awq_salient_count(K)) if n_salient is None else int(n_salient)
    nbytes = L.awq_salient_loss_workspace_bytes(N, K, T, group_size, n)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=w.device)
    idx = torch.empty(max(n, 1), dtype=torch.int32, device=w.device)[:n]
    lr, ls = np.zeros(1), np.zeros(1)
    mode = QUANT_SYMMETRIC if symmetric else QUANT_ASYMMETRIC
    st = L.awq_salient_loss(_ptr(w), _ptr(x), N, K, T, group_size, mode, n, _ptr(workspace), workspace.numel(),
                            lr.ctypes.data_as(ctypes.c_void_p), ls.ctypes.data_as(ctypes.c_void_p), _ptr(idx),
                            _stream(w.device))
    _check("awq_salient_loss", st)
    return float(lr[0]), float(ls[0]), idx


# ---------------------------------------------------------------- W8A16

def awq_quantize_w8(w, group_size: int = 128, channel_scale=None, symmetric: bool = False, out=None):
    """awq_quantize_w8: (qweight int32 [N, K/4] holding the uint32 words,
    scales fp16 [N, K/G], zeros fp16 [N, K/G])."""
    torch = _torch()
    _need_gpu("w", w, torch.float16)
    N, K = w.shape
    if channel_scale is not None:
        _need_gpu("channel_scale", channel_scale, torch.float32)
        if channel_scale.numel() != K:
            raise ValueError("channel_scale must have K elements")
    ng = K // group_size if group_size > 0 else 0
    if out is None:
        out = (torch.empty((N, max(K // 4, 0)), dtype=torch.int32, device=w.device),
               torch.empty((N, ng), dtype=torch.float16, device=w.device),
               torch.empty((N, ng), dtype=torch.float16, device=w.device))
    qweight, scales, zeros = out
    _need_out(qweight, scales, zeros, (N, K // 4), (N, ng), w.device)
    mode = QUANT_SYMMETRIC if symmetric else QUANT_ASYMMETRIC
    st = load().awq_quantize_w8(_ptr(w), _ptr(channel_scale), N, K, group_size, mode, _ptr(qweight), _ptr(scales),
                                _ptr(zeros), _stream(w.device))
    _check("awq_quantize_w8", st)
    return qweight, scales, zeros


def awq_gemm_w8(x, qweight, scales, zeros, group_size: int = 128, path: int = PATH_AUTO, out=None, workspace=None):
    """awq_gemm_w8: y = x . dequant(Wq)^T for the W8 form (path 0 auto,
    1 GEMV, 2 GEMM)."""
    torch = _torch()
    _need_gpu("x", x, torch.float16)
    _need_gpu("qweight", qweight, torch.int32)
    _need_gpu("scales", scales, torch.float16)
    _need_gpu("zeros", zeros, torch.float16)
    M, K = x.shape
    N = qweight.shape[0]
    if qweight.shape != (N, K // 4) or K % 4:
        raise ValueError("qweight must be [N, K/4]")
    if scales.shape != (N, K // group_size) or zeros.shape != scales.shape:
        raise ValueError("scales/zeros must be [N, K/group_size]")
    y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=x.device)
    _need_gpu("out", y, torch.float16)
    if tuple(y.shape) != (M, N):
        raise ValueError("out must be [M, N]")
    if workspace is not None:
        _need_gpu("workspace", workspace, torch.uint8)
    nbytes = workspace.numel() if workspace is not None else 0
    st = load().awq_gemm_w8(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(zeros), M, N, K, group_size, _ptr(y), path,
                            _ptr(workspace), nbytes, _stream(x.device))
    _check("awq_gemm_w8", st)
    return y
