"""ctypes binding of libhxq: argument marshalling only.

Every function here checks tensor shapes and dtypes on the host, takes the raw
device pointers and the current HIP stream, and calls the C entry point of the
same name.  All arithmetic happens in the library's kernels; when the library
is missing the calls raise instead of computing anything else.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

from ._digest import source_digest

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhxq.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "hxq.h")
CSRC_DIR = os.path.join(HERE, "csrc")

HXQ_OK = 0
HXQ_ERR_NULL = -1
HXQ_ERR_SHAPE = -2
HXQ_ERR_DTYPE = -3
HXQ_ERR_ALIGN = -4
HXQ_ERR_UNSUPPORTED = -5
HXQ_ERR_HIP = -6
HXQ_ERR_SCRATCH = -7
HXQ_SCRATCH_BYTES = 96 * 1024 * 1024

HXQ_F32 = 0
HXQ_BF16 = 1

HXQ_VARIANT_AUTO = 0
HXQ_VARIANT_GEMV_VALU = 1
HXQ_VARIANT_GEMV_MFMA = 2
HXQ_VARIANT_GEMM_BF16 = 3
HXQ_VARIANT_GENERIC = 4
HXQ_VARIANT_GEMM_BF16_T256 = 5

HXQ_FMT_U8 = 0
HXQ_FMT_PK12 = 1
HXQ_MAX_GROUP = 8

VARIANT_NAMES = {
    HXQ_VARIANT_AUTO: "auto",
    HXQ_VARIANT_GEMV_VALU: "gemv_valu",
    HXQ_VARIANT_GEMV_MFMA: "gemv_mfma",
    HXQ_VARIANT_GEMM_BF16: "gemm_bf16",
    HXQ_VARIANT_GENERIC: "generic",
    HXQ_VARIANT_GEMM_BF16_T256: "gemm_bf16_t256",
}


class HxqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (what, status_str(status), status))


_lib: Optional[ctypes.CDLL] = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int

class HxqLayer(ctypes.Structure):
    """struct hxq_layer of include/hxq.h."""

    _fields_ = [("codebook", ctypes.c_void_p), ("indices", ctypes.c_void_p),
                ("sc_rows", ctypes.c_void_p), ("sc_cols", ctypes.c_void_p),
                ("sc_deltas", ctypes.c_void_p), ("nnz", ctypes.c_int64),
                ("bias", ctypes.c_void_p), ("y", ctypes.c_void_p), ("N", ctypes.c_int64)]


class HxqBwdLayer(ctypes.Structure):
    """struct hxq_bwd_layer of include/hxq.h."""

    _fields_ = [("codebook", ctypes.c_void_p), ("indices", ctypes.c_void_p),
                ("sc_rows", ctypes.c_void_p), ("sc_cols", ctypes.c_void_p),
                ("sc_deltas", ctypes.c_void_p), ("nnz", ctypes.c_int64),
                ("dy", ctypes.c_void_p), ("N", ctypes.c_int64)]


_FWD_ARGS = [_P, _P, _P, _P, _P, _I64, _P, _INT, _P, _P, _I64, _I64, _I64, _P]
SIGNATURES = {
    "hxq_linear_fwd_u8": (_INT, _FWD_ARGS),
    "hxq_linear_fwd_pk12": (_INT, _FWD_ARGS),
    "hxq_linear_fwd_u8_ex": (_INT, _FWD_ARGS + [_INT]),
    "hxq_linear_fwd_pk12_ex": (_INT, _FWD_ARGS + [_INT]),
    "hxq_sidecar_add": (_INT, [_P, _P, _P, _I64, _P, _INT, _P, _I64, _I64, _I64, _P]),
    "hxq_linear_fwd_ws": (_INT, [_INT, _P, _P, _P, _P, _P, _I64, _P, _INT, _P, _P, _I64, _I64, _I64, _P, _I64, _P]),
    "hxq_linear_fwd_workspace": (_I64, [_INT, _INT, _I64, _I64, _I64]),
    "hxq_linear_fwd_grouped": (_INT, [_INT, ctypes.POINTER(HxqLayer), _INT, _P, _INT, _I64, _I64, _P]),
    "hxq_stream_read": (_INT, [_P, _I64, _P, _INT, _P]),
    "hxq_stream_read_nt": (_INT, [_P, _I64, _P, _INT, _P]),
    "hxq_dequant_bf16": (_INT, [_INT, _P, _P, _P, _P, _P, _I64, _P, _I64, _I64, _P]),
    "hxq_linear_bwd_x": (_INT, [_INT, _P, _P, _P, _P, _P, _I64, _P, _INT, _P, _I64, _I64, _I64, _P, _I64, _P]),
    "hxq_linear_bwd_x_ex": (_INT, [_INT, _P, _P, _P, _P, _P, _I64, _P, _INT, _P, _I64, _I64, _I64, _P, _I64, _P,
                                   _INT]),
    "hxq_linear_bwd_x_noalloc": (_INT, [_INT, _P, _P, _P, _P, _P, _I64, _P, _INT, _P, _I64, _I64, _I64, _P]),
    "hxq_linear_bwd_x_workspace": (_I64, [_INT, _INT, _I64, _I64, _I64, _I64]),
    "hxq_linear_bwd_x_grouped": (_INT, [_INT, ctypes.POINTER(HxqBwdLayer), _INT, _INT, _P, _I64, _I64, _P, _I64,
                                        _P]),
    "hxq_linear_bwd_x_grouped_workspace": (_I64, [_INT, _INT, ctypes.POINTER(HxqBwdLayer), _INT, _I64, _I64]),
    "hxq_select_variant": (_INT, [_INT, _INT, _I64, _I64, _I64]),
    "hxq_status_str": (ctypes.c_char_p, [_INT]),
    "hxq_version": (_INT, []),
    "hxq_source_digest": (ctypes.c_char_p, []),
}


def header_symbols(path: str = HEADER):
    """Names of the functions include/hxq.h declares."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hxq_\w+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built, or if it was built
    from sources other than the ones in the tree (rebuild it then: a process
    that has used the GPU should not compile and reload it itself)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libhxq.so is not built (%s); run python -m vq_compressed_linear_amd.build"
                               % LIB_PATH)
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        built = handle.hxq_source_digest().decode()
        if os.path.isdir(CSRC_DIR):
            want = source_digest()
            if built != want:
                raise RuntimeError("libhxq.so was built from other sources (digest %s, sources %s); "
                                   "rebuild it with python -m vq_compressed_linear_amd.build" % (built, want))
        _lib = handle
    return _lib


def status_str(status: int) -> str:
    try:
        return lib().hxq_status_str(status).decode()
    except Exception:  # the library itself could not be loaded
        return "status %d" % status


# ------------------------------------------------------------ torch marshalling

def _torch():
    import torch

    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream, dev=None) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _x_dtype(x) -> int:
    torch = _torch()
    if x.dtype == torch.float32:
        return HXQ_F32
    if x.dtype == torch.bfloat16:
        return HXQ_BF16
    raise TypeError("x must be float32 or bfloat16, got %s" % x.dtype)


def _check_device(*tensors):
    """Every tensor given (None skipped) must live on one GPU: the kernels read
    raw device pointers, and a host tensor's pointer would fault them."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("every tensor must be on a GPU; got one on %s" % t.device)
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors on different devices: %s and %s" % (dev, t.device))
    return dev


def _check_sidecar(sc_rows, sc_cols, sc_deltas):
    torch = _torch()
    if sc_rows is None:
        return 0
    if sc_rows.dtype != torch.int32 or sc_cols.dtype != torch.int32 or sc_deltas.dtype != torch.float32:
        raise TypeError("sidecar rows/cols must be int32 and deltas float32")
    nnz = sc_rows.numel()
    if sc_cols.numel() != nnz or sc_deltas.numel() != nnz:
        raise ValueError("sidecar arrays differ in length")
    for t in (sc_rows, sc_cols, sc_deltas):
        if not t.is_contiguous():
            raise ValueError("sidecar arrays must be contiguous")
    return nnz


def _check_common(x, bias, y, N):
    torch = _torch()
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [M, K] tensor")
    M, K = x.shape
    if y.dtype != torch.float32 or tuple(y.shape) != (M, N) or not y.is_contiguous():
        raise ValueError("y must be a contiguous float32 [M, N] tensor")
    if bias is not None and (bias.dtype != torch.float32 or bias.numel() != N or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous float32 [N] tensor")
    return M, K


def hxq_linear_fwd_u8(codebook, indices, sc_rows, sc_cols, sc_deltas, x, bias, y,
                      stream=None, variant: int = HXQ_VARIANT_AUTO) -> None:
    """y <- (C[indices] + S) x^T + bias on the device (u8 format)."""
    torch = _torch()
    if codebook.dtype != torch.float32 or codebook.numel() != 256:
        raise ValueError("codebook must be 256 float32 values")
    if indices.dtype != torch.uint8 or indices.dim() != 2 or not indices.is_contiguous():
        raise ValueError("indices must be a contiguous uint8 [N, K] tensor")
    N, K = indices.shape
    M, Kx = _check_common(x, bias, y, N)
    if Kx != K:
        raise ValueError("x has K=%d, indices K=%d" % (Kx, K))
    nnz = _check_sidecar(sc_rows, sc_cols, sc_deltas)
    dev = _check_device(codebook, indices, sc_rows, sc_cols, sc_deltas, x, bias, y)
    st = lib().hxq_linear_fwd_u8_ex(
        _ptr(codebook), _ptr(indices), _ptr(sc_rows), _ptr(sc_cols), _ptr(sc_deltas), nnz,
        _ptr(x), _x_dtype(x), _ptr(bias), _ptr(y), M, N, K, _stream(stream, dev), variant)
    if st != HXQ_OK:
        raise HxqError(st, "hxq_linear_fwd_u8")


def hxq_linear_fwd_pk12(codebook2, packed, sc_rows, sc_cols, sc_deltas, x, bias, y,
                        stream=None, variant: int = HXQ_VARIANT_AUTO) -> None:
    """y <- (C2[unpack(packed)] + S) x^T + bias on the device (pk12 format)."""
    torch = _torch()
    if codebook2.dtype != torch.float32 or codebook2.numel() != 4096 * 2:
        raise ValueError("codebook2 must be 4096 x 2 float32 values")
    if packed.dtype != torch.uint8 or packed.dim() != 2 or not packed.is_contiguous():
        raise ValueError("packed must be a contiguous uint8 [N, 3*ceil(K/4)] tensor")
    N = packed.shape[0]
    M, K = _check_common(x, bias, y, N)
    if packed.shape[1] != 3 * ((K + 3) // 4):
        raise ValueError("packed rows must hold 3*ceil(K/4) = %d bytes" % (3 * ((K + 3) // 4)))
    nnz = _check_sidecar(sc_rows, sc_cols, sc_deltas)
    dev = _check_device(codebook2, packed, sc_rows, sc_cols, sc_deltas, x, bias, y)
    st = lib().hxq_linear_fwd_pk12_ex(
        _ptr(codebook2), _ptr(packed), _ptr(sc_rows), _ptr(sc_cols), _ptr(sc_deltas), nnz,
        _ptr(x), _x_dtype(x), _ptr(bias), _ptr(y), M, N, K, _stream(stream, dev), variant)
    if st != HXQ_OK:
        raise HxqError(st, "hxq_linear_fwd_pk12")


def hxq_linear_fwd_ws(fmt: int, codebook, indices, sc_rows, sc_cols, sc_deltas, x, bias, y, K: int,
                      stream=None, workspace=None) -> None:
    """The forward of either format with a workspace for the k split of
    layers with few output tiles (see include/hxq.h).  K is the layer's input
    width (pk12 rows hold 3*ceil(K/4) bytes).  ``workspace`` (a device
    tensor): when None, one of the size the library asks for is taken from
    torch's caching allocator; an empty tensor means none."""
    torch = _torch()
    if fmt == HXQ_FMT_U8:
        if codebook.dtype != torch.float32 or codebook.numel() != 256:
            raise ValueError("codebook must be 256 float32 values")
        row = K
    else:
        if codebook.dtype != torch.float32 or codebook.numel() != 4096 * 2:
            raise ValueError("codebook2 must be 4096 x 2 float32 values")
        row = 3 * ((K + 3) // 4)
    if indices.dtype != torch.uint8 or indices.dim() != 2 or not indices.is_contiguous() or indices.shape[1] != row:
        raise ValueError("indices must be a contiguous uint8 [N, %d] tensor" % row)
    N = indices.shape[0]
    M, Kx = _check_common(x, bias, y, N)
    if Kx != K:
        raise ValueError("x has K=%d, the layer K=%d" % (Kx, K))
    nnz = _check_sidecar(sc_rows, sc_cols, sc_deltas)
    dev = _check_device(codebook, indices, sc_rows, sc_cols, sc_deltas, x, bias, y,
                        workspace if workspace is not None and workspace.numel() > 0 else None)
    if workspace is None:
        need = lib().hxq_linear_fwd_workspace(fmt, _x_dtype(x), M, N, K)
        if need < 0:
            raise HxqError(int(need), "hxq_linear_fwd_workspace")
        workspace = torch.empty(int(need), dtype=torch.uint8, device=y.device) if need > 0 else None
    if workspace is None or workspace.numel() == 0:
        wptr, wbytes = None, 0
    else:
        wptr, wbytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    st = lib().hxq_linear_fwd_ws(fmt, _ptr(codebook), _ptr(indices), _ptr(sc_rows), _ptr(sc_cols),
                                 _ptr(sc_deltas), nnz, _ptr(x), _x_dtype(x), _ptr(bias), _ptr(y), M, N, K,
                                 wptr, wbytes, _stream(stream, dev))
    if st != HXQ_OK:
        raise HxqError(st, "hxq_linear_fwd_ws")


def hxq_sidecar_add(sc_rows, sc_cols, sc_deltas, x, y, stream=None) -> None:
    """y <- y + S x^T on the device."""
    nnz = _check_sidecar(sc_rows, sc_cols, sc_deltas)
    N = y.shape[1]
    M, K = _check_common(x, None, y, N)
    dev = _check_device(sc_rows, sc_cols, sc_deltas, x, y)
    st = lib().hxq_sidecar_add(_ptr(sc_rows), _ptr(sc_cols), _ptr(sc_deltas), nnz, _ptr(x),
                               _x_dtype(x), _ptr(y), M, N, K, _stream(stream, dev))
    if st != HXQ_OK:
        raise HxqError(st, "hxq_sidecar_add")


def hxq_dequant_bf16(fmt: int, codebook, indices, sc_rows, sc_cols, sc_deltas, w, stream=None) -> None:
    """w <- bf16(C[indices] + S) on the device: the dense weight, for timing
    the buffered design only (the forward entry points never form it).  w is
    a contiguous [N, K] bfloat16 (or int16 / uint16 bit pattern) tensor."""
    torch = _torch()
    if w.dim() != 2 or w.element_size() != 2 or not w.is_contiguous():
        raise ValueError("w must be a contiguous [N, K] tensor of 16-bit elements")
    N, K = w.shape
    if indices.dtype != torch.uint8 or indices.dim() != 2 or not indices.is_contiguous() or indices.shape[0] != N:
        raise ValueError("indices must be a contiguous uint8 [N, row bytes] tensor")
    row = K if fmt == HXQ_FMT_U8 else 3 * ((K + 3) // 4)
    if indices.shape[1] != row:
        raise ValueError("index rows hold %d bytes, expected %d" % (indices.shape[1], row))
    if codebook.dtype != torch.float32 or codebook.numel() != (256 if fmt == HXQ_FMT_U8 else 8192):
        raise ValueError("wrong codebook size or dtype")
    nnz = _check_sidecar(sc_rows, sc_cols, sc_deltas)
    dev = _check_device(codebook, indices, sc_rows, sc_cols, sc_deltas, w)
    st = lib().hxq_dequant_bf16(fmt, _ptr(codebook), _ptr(indices), _ptr(sc_rows), _ptr(sc_cols),
                                _ptr(sc_deltas), nnz, _ptr(w), N, K, _stream(stream, dev))
    if st != HXQ_OK:
        raise HxqError(st, "hxq_dequant_bf16")


def hxq_linear_bwd_x(fmt: int, codebook, indices, sc_rows, sc_cols, sc_deltas, dy, dx, K: int,
                     stream=None, variant: int = HXQ_VARIANT_AUTO, workspace=None) -> None:
    """dx <- dy (C[indices] + S) on the device: the input gradient of a frozen
    layer.  dy is a contiguous float32 or bfloat16 [M, N] tensor, dx a
    contiguous float32 [M, K] tensor; K is the layer's input width (pk12 rows
    hold 3*ceil(K/4) bytes).  ``workspace`` (a device tensor) holds the partial
    sums of split rows; when None, one of the size the library asks for is
    taken from torch's caching allocator; an empty tensor means none."""
    torch = _torch()
    if codebook.dtype != torch.float32 or codebook.numel() != (256 if fmt == HXQ_FMT_U8 else 8192):
        raise ValueError("wrong codebook size or dtype")
    if indices.dtype != torch.uint8 or indices.dim() != 2 or not indices.is_contiguous():
        raise ValueError("indices must be a contiguous uint8 matrix")
    N = indices.shape[0]
    row = K if fmt == HXQ_FMT_U8 else 3 * ((K + 3) // 4)
    if indices.shape[1] != row:
        raise ValueError("index rows hold %d bytes, expected %d" % (indices.shape[1], row))
    if dy.dim() != 2 or not dy.is_contiguous() or dy.shape[1] != N:
        raise ValueError("dy must be a contiguous [M, N] tensor")
    M = dy.shape[0]
    if dx.dtype != torch.float32 or tuple(dx.shape) != (M, K) or not dx.is_contiguous():
        raise ValueError("dx must be a contiguous float32 [M, K] tensor")
    nnz = _check_sidecar(sc_rows, sc_cols, sc_deltas)
    dev = _check_device(codebook, indices, sc_rows, sc_cols, sc_deltas, dy, dx,
                        workspace if workspace is not None and workspace.numel() > 0 else None)
    if workspace is None:
        need = lib().hxq_linear_bwd_x_workspace(fmt, _x_dtype(dy), M, N, K, nnz)
        if need < 0:
            raise HxqError(int(need), "hxq_linear_bwd_x_workspace")
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dx.device) if need > 0 else None
    if workspace is None or workspace.numel() == 0:
        wptr, wbytes = None, 0
    else:
        wptr, wbytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    st = lib().hxq_linear_bwd_x_ex(fmt, _ptr(codebook), _ptr(indices), _ptr(sc_rows), _ptr(sc_cols),
                                   _ptr(sc_deltas), nnz, _ptr(dy), _x_dtype(dy), _ptr(dx), M, N, K,
                                   wptr, wbytes, _stream(stream, dev), variant)
    if st != HXQ_OK:
        raise HxqError(st, "hxq_linear_bwd_x")


def hxq_linear_bwd_x_noalloc(fmt: int, codebook, indices, sc_rows, sc_cols, sc_deltas, dy, dx, K: int,
                             stream=None) -> None:
    """dx <- dy (C[indices] + S), like hxq_linear_bwd_x, with the library's own
    device scratch instead of a workspace (nothing is allocated, here or in
    the library).  Calls that overlap on one GPU race on that scratch."""
    torch = _torch()
    if codebook.dtype != torch.float32 or codebook.numel() != (256 if fmt == HXQ_FMT_U8 else 8192):
        raise ValueError("wrong codebook size or dtype")
    if indices.dtype != torch.uint8 or indices.dim() != 2 or not indices.is_contiguous():
        raise ValueError("indices must be a contiguous uint8 matrix")
    N = indices.shape[0]
    row = K if fmt == HXQ_FMT_U8 else 3 * ((K + 3) // 4)
    if indices.shape[1] != row:
        raise ValueError("index rows hold %d bytes, expected %d" % (indices.shape[1], row))
    if dy.dim() != 2 or not dy.is_contiguous() or dy.shape[1] != N:
        raise ValueError("dy must be a contiguous [M, N] tensor")
    M = dy.shape[0]
    if dx.dtype != torch.float32 or tuple(dx.shape) != (M, K) or not dx.is_contiguous():
        raise ValueError("dx must be a contiguous float32 [M, K] tensor")
    nnz = _check_sidecar(sc_rows, sc_cols, sc_deltas)
    dev = _check_device(codebook, indices, sc_rows, sc_cols, sc_deltas, dy, dx)
    st = lib().hxq_linear_bwd_x_noalloc(fmt, _ptr(codebook), _ptr(indices), _ptr(sc_rows), _ptr(sc_cols),
                                        _ptr(sc_deltas), nnz, _ptr(dy), _x_dtype(dy), _ptr(dx), M, N, K,
                                        _stream(stream, dev))
    if st != HXQ_OK:
        raise HxqError(st, "hxq_linear_bwd_x_noalloc")


def grouped_layers(fmt: int, layers, M: int, K: int, x=None):
    """HxqLayer array for hxq_linear_fwd_grouped from dicts holding the
    tensors codebook, indices, sc_rows, sc_cols, sc_deltas, bias (or None) and
    y.  Checks dtypes and shapes like the single-layer functions."""
    torch = _torch()
    if not 1 <= len(layers) <= HXQ_MAX_GROUP:
        raise ValueError("between 1 and %d layers per call" % HXQ_MAX_GROUP)
    arr = (HxqLayer * len(layers))()
    for i, l in enumerate(layers):
        cb, idx, y, bias = l["codebook"], l["indices"], l["y"], l.get("bias")
        if cb.dtype != torch.float32 or cb.numel() != (256 if fmt == HXQ_FMT_U8 else 8192):
            raise ValueError("layer %d: wrong codebook size or dtype" % i)
        if idx.dtype != torch.uint8 or idx.dim() != 2 or not idx.is_contiguous():
            raise ValueError("layer %d: indices must be a contiguous uint8 matrix" % i)
        N = idx.shape[0]
        row = K if fmt == HXQ_FMT_U8 else 3 * ((K + 3) // 4)
        if idx.shape[1] != row:
            raise ValueError("layer %d: index rows hold %d bytes, expected %d" % (i, idx.shape[1], row))
        if y.dtype != torch.float32 or tuple(y.shape) != (M, N) or not y.is_contiguous():
            raise ValueError("layer %d: y must be a contiguous float32 [M, N] tensor" % i)
        if bias is not None and (bias.dtype != torch.float32 or bias.numel() != N):
            raise ValueError("layer %d: bias must be float32 [N]" % i)
        nnz = _check_sidecar(l.get("sc_rows"), l.get("sc_cols"), l.get("sc_deltas"))
        _check_device(x, cb, idx, l.get("sc_rows"), l.get("sc_cols"), l.get("sc_deltas"), bias, y)
        arr[i] = HxqLayer(_ptr(cb), _ptr(idx), _ptr(l.get("sc_rows")), _ptr(l.get("sc_cols")),
                          _ptr(l.get("sc_deltas")), nnz, _ptr(bias), _ptr(y), N)
    return arr


def hxq_linear_fwd_grouped(fmt: int, layers, x, stream=None) -> None:
    """Each layer's y <- (codebook[indices] + S) x^T + bias, all from one x."""
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [M, K] tensor")
    M, K = x.shape
    arr = grouped_layers(fmt, layers, M, K, x)
    dev = _check_device(x)
    st = lib().hxq_linear_fwd_grouped(fmt, arr, len(layers), _ptr(x), _x_dtype(x), M, K, _stream(stream, dev))
    if st != HXQ_OK:
        raise HxqError(st, "hxq_linear_fwd_grouped")


def grouped_bwd_layers(fmt: int, layers, M: int, K: int, dy_dtype: int):
    """HxqBwdLayer array for hxq_linear_bwd_x_grouped from dicts holding the
    tensors codebook, indices, sc_rows, sc_cols, sc_deltas (or None) and dy.
    Checks dtypes and shapes like hxq_linear_bwd_x."""
    torch = _torch()
    if not 1 <= len(layers) <= HXQ_MAX_GROUP:
        raise ValueError("between 1 and %d layers per call" % HXQ_MAX_GROUP)
    arr = (HxqBwdLayer * len(layers))()
    for i, l in enumerate(layers):
        cb, idx, dy = l["codebook"], l["indices"], l["dy"]
        if cb.dtype != torch.float32 or cb.numel() != (256 if fmt == HXQ_FMT_U8 else 8192):
            raise ValueError("layer %d: wrong codebook size or dtype" % i)
        if idx.dtype != torch.uint8 or idx.dim() != 2 or not idx.is_contiguous():
            raise ValueError("layer %d: indices must be a contiguous uint8 matrix" % i)
        N = idx.shape[0]
        row = K if fmt == HXQ_FMT_U8 else 3 * ((K + 3) // 4)
        if idx.shape[1] != row:
            raise ValueError("layer %d: index rows hold %d bytes, expected %d" % (i, idx.shape[1], row))
        if dy.dim() != 2 or not dy.is_contiguous() or tuple(dy.shape) != (M, N) or _x_dtype(dy) != dy_dtype:
            raise ValueError("layer %d: dy must be a contiguous [M, N] tensor of the group's dtype" % i)
        nnz = _check_sidecar(l.get("sc_rows"), l.get("sc_cols"), l.get("sc_deltas"))
        _check_device(cb, idx, l.get("sc_rows"), l.get("sc_cols"), l.get("sc_deltas"), dy)
        arr[i] = HxqBwdLayer(_ptr(cb), _ptr(idx), _ptr(l.get("sc_rows")), _ptr(l.get("sc_cols")),
                             _ptr(l.get("sc_deltas")), nnz, _ptr(dy), N)
    return arr


def hxq_linear_bwd_x_grouped(fmt: int, layers, dx, stream=None, workspace=None) -> None:
    """dx <- sum over layers of dy_i (C_i[indices_i] + S_i): the input gradient
    of layers that share their input (each dict as for grouped_bwd_layers).
    dx is a contiguous float32 [M, K] tensor.  ``workspace`` (a device tensor)
    holds the partial sums; when None, one of the size the library asks for
    is taken from torch's caching allocator."""
    torch = _torch()
    if dx.dtype != torch.float32 or dx.dim() != 2 or not dx.is_contiguous():
        raise ValueError("dx must be a contiguous float32 [M, K] tensor")
    M, K = dx.shape
    if not layers:
        raise ValueError("between 1 and %d layers per call" % HXQ_MAX_GROUP)
    dyt = _x_dtype(layers[0]["dy"])
    arr = grouped_bwd_layers(fmt, layers, M, K, dyt)
    dev = _check_device(dx, workspace if workspace is not None and workspace.numel() > 0 else None)
    if workspace is None:
        need = lib().hxq_linear_bwd_x_grouped_workspace(fmt, dyt, arr, len(layers), M, K)
        if need < 0:
            raise HxqError(int(need), "hxq_linear_bwd_x_grouped_workspace")
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dx.device) if need > 0 else None
    if workspace is None or workspace.numel() == 0:
        wptr, wbytes = None, 0
    else:
        wptr, wbytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    st = lib().hxq_linear_bwd_x_grouped(fmt, arr, len(layers), dyt, _ptr(dx), M, K, wptr, wbytes,
                                        _stream(stream, dev))
    if st != HXQ_OK:
        raise HxqError(st, "hxq_linear_bwd_x_grouped")


def hxq_linear_bwd_x_workspace(fmt: int, dy_dtype: int, M: int, N: int, K: int, nnz: int) -> int:
    """Bytes of workspace hxq_linear_bwd_x uses for these sizes."""
    n = lib().hxq_linear_bwd_x_workspace(fmt, dy_dtype, M, N, K, nnz)
    if n < 0:
        raise HxqError(int(n), "hxq_linear_bwd_x_workspace")
    return int(n)


def hxq_select_variant(fmt_pk12: bool, x_dtype: int, M: int, N: int, K: int) -> int:
    return lib().hxq_select_variant(int(bool(fmt_pk12)), x_dtype, M, N, K)


def hxq_version() -> int:
    return lib().hxq_version()
