"""Thin ctypes binding of libqlora (include/qlora.h), same names as the C ABI.

Argument marshalling only: every step of the computation runs in the HIP
library. PyTorch provides device memory (outputs and workspaces are
allocated here with torch) and the stream (torch's current stream).
If libqlora.so is missing, every call raises: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
# Always the in-tree build next to this file (python -m
# quantized_frozen_weight_amd.build_lib); no other copy is ever loaded.
LIB_PATH = os.path.join(HERE, "libqlora.so")

QLORA_OK, QLORA_EINVAL, QLORA_EUNSUPPORTED, QLORA_EWORKSPACE, QLORA_ERANGE, QLORA_EHIP = range(6)
QLORA_F32, QLORA_BF16 = 0, 1
QLORA_W8, QLORA_W4G128, QLORA_W8O = 0, 1, 2

_FMT = {"w8": QLORA_W8, "w4g128": QLORA_W4G128, "w8o": QLORA_W8O}


class QloraError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {qlora_status_str(status)} ({status})")


class qlora_linear(ctypes.Structure):
    _fields_ = [
        ("K", ctypes.c_int32),
        ("N", ctypes.c_int32),
        ("r", ctypes.c_int32),
        ("alpha", ctypes.c_float),
        ("fmt", ctypes.c_int32),
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("A", ctypes.c_void_p),
        ("B", ctypes.c_void_p),
        ("heads", ctypes.c_int32),
    ]


_lib = None

EXPORTS = (
    "qlora_status_str", "qlora_weight_bytes", "qlora_quantize",
    "qlora_fwd_workspace", "qlora_fwd", "qlora_bwd_workspace", "qlora_bwd",
    "qlora_quantize_rows", "qlora_fwd_acc", "qlora_fwd_timed", "qlora_bwd_timed",
    "qlora_merge", "qlora_bwd_partial", "qlora_bwd_finish", "qlora_fwd_a8w4",
    "qlora_quantize_heads", "qlora_outlier_layout", "qlora_bwd_finish_batch",
    "qlora_bwd_partials_bytes", "qlora_bwd_main_kernel", "qlora_bwd_noalloc",
)
QLORA_NOALLOC_SCRATCH_BYTES = 16 << 20
# include/qlora_probe.h: measurement probes (not part of the layer)
PROBE_EXPORTS = ("qlora_probe_mfma", "qlora_probe_copy", "qlora_probe_read", "qlora_probe_empty")
QLORA_PROBE_BF16, QLORA_PROBE_I8 = 0, 1


class qlora_finish_item(ctypes.Structure):
    _fields_ = [
        ("L", ctypes.c_void_p),
        ("M", ctypes.c_int),
        ("dtype", ctypes.c_int),
        ("dA", ctypes.c_void_p),
        ("dB", ctypes.c_void_p),
        ("ws", ctypes.c_void_p),
        ("ws_bytes", ctypes.c_size_t),
    ]


def lib() -> ctypes.CDLL:
    """Load libqlora.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m quantized_frozen_weight_amd.build_lib`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    psz = ctypes.POINTER(ctypes.c_size_t)
    plin = ctypes.POINTER(qlora_linear)
    L.qlora_status_str.argtypes = [i]
    L.qlora_status_str.restype = ctypes.c_char_p
    L.qlora_weight_bytes.argtypes = [i, i, i, psz, psz]
    L.qlora_quantize.argtypes = [vp, i, i, i, vp, vp, vp]
    L.qlora_fwd_workspace.argtypes = [plin, i, i, psz]
    L.qlora_fwd.argtypes = [plin, i, i, vp, vp, vp, vp, sz, vp]
    L.qlora_bwd_workspace.argtypes = [plin, i, i, psz]
    L.qlora_bwd.argtypes = [plin, i, i, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.qlora_quantize_rows.argtypes = [vp, i, i, i, vp, vp, vp]
    L.qlora_fwd_acc.argtypes = [plin, i, i, vp, vp, vp, sz, vp]
    L.qlora_fwd_timed.argtypes = [plin, i, i, vp, vp, vp, vp, sz, vp, i, vp, vp]
    L.qlora_bwd_timed.argtypes = [plin, i, i, vp, vp, vp, vp, vp, vp, vp, sz, vp, i, vp, vp]
    L.qlora_merge.argtypes = [plin, vp, vp, vp]
    L.qlora_bwd_partial.argtypes = [plin, i, i, vp, vp, vp, vp, vp, sz, vp]
    L.qlora_bwd_finish.argtypes = [plin, i, i, vp, vp, vp, sz, vp]
    L.qlora_bwd_finish_batch.argtypes = [ctypes.POINTER(qlora_finish_item), i, vp]
    L.qlora_bwd_partials_bytes.argtypes = [plin, i, i, psz]
    L.qlora_fwd_a8w4.argtypes = [plin, i, i, vp, vp, vp, vp, sz, vp]
    L.qlora_quantize_heads.argtypes = [vp, i, i, i, i, vp, vp, vp]
    L.qlora_outlier_layout.argtypes = [i, i, psz, psz, psz, ctypes.POINTER(ctypes.c_int32)]
    L.qlora_bwd_main_kernel.argtypes = [plin, i, i]
    L.qlora_bwd_noalloc.argtypes = [plin, i, i, vp, vp, vp, vp, vp, vp, vp]
    for name in EXPORTS[1:]:
        getattr(L, name).restype = ctypes.c_int
    L.qlora_bwd_main_kernel.restype = ctypes.c_char_p
    L.qlora_probe_mfma.argtypes = [i, i, i, vp, vp, ctypes.POINTER(ctypes.c_double)]
    L.qlora_probe_copy.argtypes = [vp, vp, sz, i, vp]
    L.qlora_probe_read.argtypes = [vp, sz, i, vp, vp]
    L.qlora_probe_empty.argtypes = [i, i, vp]
    for name in PROBE_EXPORTS:
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def loaded_path() -> str:
    """Path of the libqlora.so this process has mapped (from
    /proc/self/maps), after lib() has loaded it; '' if none is mapped."""
    lib()
    with open("/proc/self/maps") as f:
        for line in f:
            if line.rstrip().endswith("/libqlora.so"):
                return line.split()[-1]
    return ""


def qlora_bwd_main_kernel(layer: "QLinear", M: int, dtype: int) -> str:
    """Name of the kernel qlora_bwd_timed times for this layer (static)."""
    s = layer.cstruct()
    name = lib().qlora_bwd_main_kernel(ctypes.byref(s), M, dtype)
    if name is None:
        raise QloraError(QLORA_EINVAL, "qlora_bwd_main_kernel")
    return name.decode()


def _check(status: int, what: str) -> None:
    if status != QLORA_OK:
        raise QloraError(status, what)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return QLORA_F32
    if t.dtype == torch.bfloat16:
        return QLORA_BF16
    raise TypeError(f"unsupported activation dtype {t.dtype}")


def qlora_status_str(status: int) -> str:
    return lib().qlora_status_str(int(status)).decode()


def qlora_weight_bytes(K: int, N: int, fmt: str = "w8") -> Tuple[int, int]:
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().qlora_weight_bytes(K, N, _FMT[fmt], ctypes.byref(cb), ctypes.byref(sb)),
           "qlora_weight_bytes")
    return cb.value, sb.value


@dataclass
class QLinear:
    """A frozen quantized weight plus its adapter (device tensors)."""
    K: int
    N: int
    r: int
    alpha: float
    fmt: str
    codes: object     # int8 [N, K]  or uint8 [N, K/2]
    scales: object    # float32 [N], float16 [N, K/128], or the w8o side buffer (uint8)
    A: object         # float32 [K, r]
    B: object         # float32 [r, N], or [heads, r, N / heads]
    heads: int = 1

    def cstruct(self) -> qlora_linear:
        return qlora_linear(self.K, self.N, self.r, float(self.alpha), _FMT[self.fmt],
                            _ptr(self.codes), _ptr(self.scales), _ptr(self.A),
                            _ptr(self.B), int(self.heads))


def _b_shape(layer: QLinear):
    """Shape of B and dB: [r, N], or [heads, r, N / heads]."""
    if layer.heads > 1:
        return (layer.heads, layer.r, layer.N // layer.heads)
    return (layer.r, layer.N)


def qlora_quantize(W, fmt: str = "w8"):
    """W float32 [K, N], or per head [heads, K, hd] (N = heads * hd), on the
    GPU -> (codes, scales) in the library's layout."""
    import torch
    if W.dim() == 3:
        heads, K, hd = W.shape
        N = heads * hd
    else:
        heads, (K, N) = 1, W.shape
    cb, sb = qlora_weight_bytes(K, N, fmt)
    if fmt == "w8":
        codes = torch.empty((N, K), dtype=torch.int8, device=W.device)
        scales = torch.empty((N,), dtype=torch.float32, device=W.device)
    elif fmt == "w8o":
        codes = torch.empty((N, K), dtype=torch.int8, device=W.device)
        scales = torch.empty((sb,), dtype=torch.uint8, device=W.device)
    else:
        codes = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
        scales = torch.empty((N, K // 128), dtype=torch.float16, device=W.device)
    assert codes.numel() * codes.element_size() == cb
    assert scales.numel() * scales.element_size() == sb
    W = W.contiguous()
    _check(lib().qlora_quantize_heads(_ptr(W), heads, K, N, _FMT[fmt], _ptr(codes),
                                      _ptr(scales), _stream()), "qlora_quantize_heads")
    return codes, scales


def qlora_outlier_layout(K: int, N: int) -> Tuple[int, int, int, int]:
    """(rowptr, col, val) byte offsets of a w8o side buffer's outlier list,
    and its capacity."""
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    cap = ctypes.c_int32()
    _check(lib().qlora_outlier_layout(K, N, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c),
                                      ctypes.byref(cap)), "qlora_outlier_layout")
    return a.value, b.value, c.value, cap.value


def qlora_outliers(side, K: int, N: int):
    """Read a w8o side buffer back (device -> host): (header dict with lo, hi,
    scale, nnz; rowptr int32 [K + 1]; col int32 [nnz]; val float16 [nnz])."""
    import numpy as np
    ro, co, vo, _ = qlora_outlier_layout(K, N)
    raw = side.cpu().numpy()
    hdr = raw[:16].view(np.float32)
    nnz = int(raw[12:16].view(np.int32)[0])
    head = dict(lo=hdr[0], hi=hdr[1], scale=hdr[2], nnz=nnz)
    rowptr = raw[ro:ro + 4 * (K + 1)].view(np.int32).copy()
    col = raw[co:co + 4 * nnz].view(np.int32).copy()
    val = raw[vo:vo + 2 * nnz].view(np.float16).copy()
    return head, rowptr, col, val


def qlora_merge(layer: QLinear):
    """The adapter merged into the layer's int8 weight, re-quantized: new
    (codes int8 [N, K], scales float32 [N]) on the layer's device."""
    import torch
    codes = torch.empty((layer.N, layer.K), dtype=torch.int8, device=layer.codes.device)
    scales = torch.empty((layer.N,), dtype=torch.float32, device=layer.codes.device)
    s = layer.cstruct()
    _check(lib().qlora_merge(ctypes.byref(s), _ptr(codes), _ptr(scales), _stream()),
           "qlora_merge")
    return codes, scales


def qlora_fwd_workspace(layer: QLinear, M: int, dtype: int) -> int:
    n = ctypes.c_size_t()
    s = layer.cstruct()
    _check(lib().qlora_fwd_workspace(ctypes.byref(s), M, dtype, ctypes.byref(n)),
           "qlora_fwd_workspace")
    return n.value


def qlora_bwd_workspace(layer: QLinear, M: int, dtype: int) -> int:
    n = ctypes.c_size_t()
    s = layer.cstruct()
    _check(lib().qlora_bwd_workspace(ctypes.byref(s), M, dtype, ctypes.byref(n)),
           "qlora_bwd_workspace")
    return n.value


def _workspace(nbytes: int, device, ws=None):
    import torch
    if ws is not None:
        return ws
    return torch.empty((max(nbytes, 256),), dtype=torch.uint8, device=device)


def qlora_fwd(layer: QLinear, x, save_t: bool = True, y=None, t=None, ws=None):
    """y = x deq(W) + s (x A) B. Returns (y, t) (t is None if not saved)."""
    import torch
    M = x.shape[0]
    dt = _dtype_code(x)
    if y is None:
        y = torch.empty((M, layer.N), dtype=x.dtype, device=x.device)
    if save_t and t is None:
        t = torch.empty((M, layer.r), dtype=torch.float32, device=x.device)
    nbytes = qlora_fwd_workspace(layer, M, dt)
    ws = _workspace(nbytes, x.device, ws)
    s = layer.cstruct()
    _check(lib().qlora_fwd(ctypes.byref(s), M, dt, _ptr(x), _ptr(y),
                           _ptr(t) if save_t else None, _ptr(ws),
                           ws.numel() * ws.element_size(), _stream()), "qlora_fwd")
    return y, (t if save_t else None)


def qlora_fwd_a8w4(layer: QLinear, x, save_t: bool = True, y=None, t=None, ws=None):
    """Integer forward of a 4-bit layer with int8 activations: (y, t or None)."""
    import torch
    M = x.shape[0]
    dt = _dtype_code(x)
    if y is None:
        y = torch.empty((M, layer.N), dtype=x.dtype, device=x.device)
    if save_t and t is None:
        t = torch.empty((M, layer.r), dtype=torch.float32, device=x.device)
    ws = _workspace(qlora_fwd_workspace(layer, M, dt), x.device, ws)
    s = layer.cstruct()
    _check(lib().qlora_fwd_a8w4(ctypes.byref(s), M, dt, _ptr(x), _ptr(y),
                                _ptr(t) if save_t else None, _ptr(ws),
                                ws.numel() * ws.element_size(), _stream()),
           "qlora_fwd_a8w4")
    return y, (t if save_t else None)


def qlora_bwd(layer: QLinear, x, dy, t=None, need_dx: bool = True, dx=None,
              dA=None, dB=None, ws=None):
    """Returns (dx or None, dA [K, r], dB [r, N])."""
    import torch
    M = x.shape[0]
    dt = _dtype_code(x)
    if need_dx and dx is None:
        dx = torch.empty((M, layer.K), dtype=x.dtype, device=x.device)
    if dA is None:
        dA = torch.empty((layer.K, layer.r), dtype=torch.float32, device=x.device)
    if dB is None:
        dB = torch.empty(_b_shape(layer), dtype=torch.float32, device=x.device)
    nbytes = qlora_bwd_workspace(layer, M, dt)
    ws = _workspace(nbytes, x.device, ws)
    s = layer.cstruct()
    _check(lib().qlora_bwd(ctypes.byref(s), M, dt, _ptr(x), _ptr(dy), _ptr(t),
                           _ptr(dx) if need_dx else None, _ptr(dA), _ptr(dB),
                           _ptr(ws), ws.numel() * ws.element_size(), _stream()),
           "qlora_bwd")
    return (dx if need_dx else None), dA, dB


def qlora_bwd_partial(layer: QLinear, x, dy, t=None, need_dx: bool = True, dx=None,
                      ws=None, stream=None):
    """First half of qlora_bwd: dx (or None) and the adapter-gradient partial
    sums, which stay in the returned workspace for qlora_bwd_finish."""
    import torch
    M = x.shape[0]
    dt = _dtype_code(x)
    if need_dx and dx is None:
        dx = torch.empty((M, layer.K), dtype=x.dtype, device=x.device)
    ws = _workspace(qlora_bwd_workspace(layer, M, dt), x.device, ws)
    s = layer.cstruct()
    _check(lib().qlora_bwd_partial(ctypes.byref(s), M, dt, _ptr(x), _ptr(dy), _ptr(t),
                                   _ptr(dx) if need_dx else None, _ptr(ws),
                                   ws.numel() * ws.element_size(),
                                   _stream() if stream is None else stream.cuda_stream),
           "qlora_bwd_partial")
    return (dx if need_dx else None), ws


def qlora_bwd_partials_bytes(layer: QLinear, M: int, dtype: int) -> int:
    """Leading bytes of a backward workspace that outlive qlora_bwd_partial."""
    n = ctypes.c_size_t()
    s = layer.cstruct()
    _check(lib().qlora_bwd_partials_bytes(ctypes.byref(s), M, dtype, ctypes.byref(n)),
           "qlora_bwd_partials_bytes")
    return n.value


def qlora_bwd_finish_batch(items, stream=None):
    """qlora_bwd_finish for several layers in one launch (per 32 layers).
    items: (layer, M, dtype, ws) or (layer, M, dtype, ws, dA, dB) tuples, each
    ws holding that layer's qlora_bwd_partial results. The items' partial
    sums (the first qlora_bwd_partials_bytes of each ws) must not overlap;
    the scratch past them may (packed workspaces).
    Returns the list of (dA, dB)."""
    import torch
    arr = (qlora_finish_item * len(items))()
    keep, out = [], []
    for n, it in enumerate(items):
        layer, M, dtype, ws = it[:4]
        dA = it[4] if len(it) > 4 else None
        dB = it[5] if len(it) > 5 else None
        if dA is None:
            dA = torch.empty((layer.K, layer.r), dtype=torch.float32, device=ws.device)
        if dB is None:
            dB = torch.empty(_b_shape(layer), dtype=torch.float32, device=ws.device)
        s = layer.cstruct()
        keep.append(s)
        arr[n] = qlora_finish_item(ctypes.cast(ctypes.pointer(s), ctypes.c_void_p), M,
                                   QLORA_F32 if dtype == torch.float32 else QLORA_BF16,
                                   _ptr(dA), _ptr(dB), _ptr(ws), ws.numel() * ws.element_size())
        out.append((dA, dB))
    _check(lib().qlora_bwd_finish_batch(arr, len(items),
                                        _stream() if stream is None else stream.cuda_stream),
           "qlora_bwd_finish_batch")
    return out


def qlora_bwd_finish(layer: QLinear, M: int, dtype, ws, dA=None, dB=None, stream=None):
    """Second half of qlora_bwd: dA [K, r] and dB [r, N] from the partial sums
    that qlora_bwd_partial left in ws. dtype: the activations' torch dtype."""
    import torch
    dt = QLORA_F32 if dtype == torch.float32 else QLORA_BF16
    if dA is None:
        dA = torch.empty((layer.K, layer.r), dtype=torch.float32, device=ws.device)
    if dB is None:
        dB = torch.empty(_b_shape(layer), dtype=torch.float32, device=ws.device)
    s = layer.cstruct()
    _check(lib().qlora_bwd_finish(ctypes.byref(s), M, dt, _ptr(dA), _ptr(dB), _ptr(ws),
                                  ws.numel() * ws.element_size(),
                                  _stream() if stream is None else stream.cuda_stream),
           "qlora_bwd_finish")
    return dA, dB


def qlora_quantize_rows(x):
    """Test hook: (xq int8 [M, K], sx float32 [M]) from the forward's quantizer."""
    import torch
    M, K = x.shape
    xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    sx = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(lib().qlora_quantize_rows(_ptr(x), M, K, _dtype_code(x), _ptr(xq), _ptr(sx),
                                     _stream()), "qlora_quantize_rows")
    return xq, sx


def qlora_fwd_acc(layer: QLinear, x):
    """Test hook: exact int32 product of the quantized rows and codes [M, N]."""
    import torch
    M = x.shape[0]
    dt = _dtype_code(x)
    acc = torch.empty((M, layer.N), dtype=torch.int32, device=x.device)
    ws = _workspace(qlora_fwd_workspace(layer, M, dt), x.device)
    s = layer.cstruct()
    _check(lib().qlora_fwd_acc(ctypes.byref(s), M, dt, _ptr(x), _ptr(acc), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream()),
           "qlora_fwd_acc")
    return acc
