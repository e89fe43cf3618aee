"""Thin Python binding of libsbl (include/sbl.h) over PyTorch device tensors.

Argument marshalling only: every step of the path runs in the HIP kernels of
libsbl.so.  PyTorch supplies device memory and the current HIP stream.  The
binding checks that each tensor is on the GPU, contiguous, of the right dtype
and large enough for the sizes passed, so a kernel can never be handed a
buffer smaller than it will touch.  There is no CPU fallback: if the library
is missing, loading fails loudly.
"""

from __future__ import annotations

import ctypes
import os

import torch  # loaded first so libsbl binds to the same HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsbl.so")

SBL_OK = 0
SBL_FMT_DENSE2 = 0
SBL_FMT_NM = 1
# weight-preparation variants and execution choices (sbl_quant_weights_batch_ex flags)
SBL_QW_DEFAULT, SBL_QW_BETA_KEPT, SBL_QW_MASK_FROM_CODES = 0, 1, 2
SBL_QW_TWO_PASS, SBL_QW_NO_WAIT = 4, 8
ABI_VERSION = 11

_c_i64 = ctypes.c_int64
_c_i32 = ctypes.c_int32
_c_p = ctypes.c_void_p

_lib = None


class LinearItem(ctypes.Structure):
    """sbl_linear_item of include/sbl.h."""
    _fields_ = [("packed", _c_p), ("meta", _c_p), ("beta", _c_p), ("xq", _c_p), ("gamma", _c_p),
                ("m_tok", _c_i64), ("n_out", _c_i64), ("k", _c_i64), ("y", _c_p), ("acc", _c_p)]


class QuantItem(ctypes.Structure):
    """sbl_quant_item of include/sbl.h."""
    _fields_ = [("w_bf16", _c_p), ("n_out", _c_i64), ("k", _c_i64), ("beta", _c_p),
                ("mask_bits", _c_p), ("codes", _c_p), ("packed", _c_p), ("meta", _c_p),
                ("workspace", _c_p), ("workspace_bytes", _c_i64)]


class SblError(RuntimeError):
    def __init__(self, func: str, status: int):
        lib = load()
        msg = lib.sbl_status_string(status).decode()
        if status == 5:
            msg += f" (hip error {lib.sbl_last_hip_error()})"
        super().__init__(f"{func}: status {status}: {msg}")
        self.status = status


def load():
    """Load libsbl.so (built in-tree by build.py / __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    lib.sbl_abi_version.restype = ctypes.c_int
    lib.sbl_status_string.restype = ctypes.c_char_p
    lib.sbl_status_string.argtypes = [ctypes.c_int]
    lib.sbl_last_hip_error.restype = ctypes.c_int
    lib.sbl_packed_bytes.restype = _c_i64
    lib.sbl_packed_bytes.argtypes = [_c_i64, _c_i64, _c_i32, _c_i32, _c_i32]
    lib.sbl_meta_bytes.restype = _c_i64
    lib.sbl_meta_bytes.argtypes = [_c_i64, _c_i64, _c_i32]
    lib.sbl_workspace_bytes.restype = _c_i64
    lib.sbl_workspace_bytes.argtypes = [_c_i64, _c_i64]
    lib.sbl_workspace_init.restype = ctypes.c_int
    lib.sbl_workspace_init.argtypes = [_c_p, _c_i64, _c_p]
    lib.sbl_quant_weights.restype = ctypes.c_int
    lib.sbl_quant_weights.argtypes = [_c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_p, _c_p, _c_p,
                                      _c_i32, _c_p, _c_p, _c_p, _c_i64, _c_p]
    lib.sbl_quant_weights_batch.restype = ctypes.c_int
    lib.sbl_quant_weights_batch.argtypes = [ctypes.POINTER(QuantItem), _c_i32, _c_i32, _c_i32, _c_i32,
                                            _c_p]
    lib.sbl_quant_weights_batch_ex.restype = ctypes.c_int
    lib.sbl_quant_weights_batch_ex.argtypes = [ctypes.POINTER(QuantItem), _c_i32, _c_i32, _c_i32, _c_i32,
                                               _c_i32, _c_p]
    lib.sbl_quant_weights_batch_noalloc.restype = ctypes.c_int
    lib.sbl_quant_weights_batch_noalloc.argtypes = [ctypes.POINTER(QuantItem), _c_i32, _c_i32, _c_i32, _c_i32,
                                                    _c_p]
    lib.sbl_pack.restype = ctypes.c_int
    lib.sbl_pack.argtypes = [_c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_p, _c_p, _c_p]
    lib.sbl_quant_acts.restype = ctypes.c_int
    lib.sbl_quant_acts.argtypes = [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p]
    lib.sbl_linear.restype = ctypes.c_int
    lib.sbl_linear.argtypes = [_c_p, _c_p, _c_i32, _c_i32, _c_i32, _c_p, _c_p, _c_p,
                               _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p]
    lib.sbl_linear_batch.restype = ctypes.c_int
    lib.sbl_linear_batch.argtypes = [ctypes.POINTER(LinearItem), _c_i32, _c_i32, _c_i32, _c_i32, _c_p]
    lib.sbl_linear_acts_batch.restype = ctypes.c_int
    lib.sbl_linear_acts_batch.argtypes = [_c_p, _c_i64, _c_i64, _c_p, _c_p, ctypes.POINTER(LinearItem),
                                          _c_i32, _c_i32, _c_i32, _c_i32, _c_p]
    lib.sbl_workspace_bytes_grouped.restype = _c_i64
    lib.sbl_workspace_bytes_grouped.argtypes = [_c_i64, _c_i64, _c_i64]
    lib.sbl_quant_weights_grouped.restype = ctypes.c_int
    lib.sbl_quant_weights_grouped.argtypes = [_c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i64, _c_p, _c_p, _c_p,
                                              _c_i32, _c_p, _c_p, _c_p, _c_i64, _c_p]
    lib.sbl_linear_grouped.restype = ctypes.c_int
    lib.sbl_linear_grouped.argtypes = [_c_p, _c_p, _c_i32, _c_i32, _c_i32, _c_p, _c_i64, _c_p, _c_p,
                                       _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p]
    lib.sbl_quant_acts_kgrouped.restype = ctypes.c_int
    lib.sbl_quant_acts_kgrouped.argtypes = [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p]
    lib.sbl_workspace_bytes_blocked.restype = _c_i64
    lib.sbl_workspace_bytes_blocked.argtypes = [_c_i64, _c_i64, _c_i64, _c_i64]
    lib.sbl_quant_weights_blocked.restype = ctypes.c_int
    lib.sbl_quant_weights_blocked.argtypes = [_c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i64, _c_i64, _c_p, _c_p, _c_p,
                                              _c_i32, _c_p, _c_p, _c_p, _c_i64, _c_p]
    lib.sbl_linear_blocked.restype = ctypes.c_int
    lib.sbl_linear_blocked.argtypes = [_c_p, _c_p, _c_i32, _c_i32, _c_i32, _c_p, _c_i64, _c_p, _c_p, _c_i64,
                                       _c_i64, _c_i64, _c_i64, _c_p, _c_p]
    lib.sbl_linear_kgrouped.restype = ctypes.c_int
    lib.sbl_linear_kgrouped.argtypes = [_c_p, _c_p, _c_i32, _c_i32, _c_i32, _c_p, _c_i64, _c_p, _c_p, _c_i64,
                                        _c_i64, _c_i64, _c_i64, _c_p, _c_p]
    lib.sbl_linear_backward.restype = ctypes.c_int
    lib.sbl_linear_backward.argtypes = [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_i32, _c_i32, _c_i32,
                                        _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p]
    lib.sbl_backward_workspace_bytes.restype = ctypes.c_int64
    lib.sbl_backward_workspace_bytes.argtypes = [_c_i64, _c_i64, _c_i64]
    lib.sbl_linear_backward_ws.restype = ctypes.c_int
    lib.sbl_linear_backward_ws.argtypes = [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_i32, _c_i32, _c_i32,
                                           _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_p]
    if lib.sbl_abi_version() != ABI_VERSION:
        raise RuntimeError("libsbl.so ABI version mismatch: rebuild it")
    _lib = lib
    return lib


# ---------------------------------------------------------------- helpers

def _ptr(t, dtype, nbytes: int, name: str):
    """Device pointer of a contiguous tensor holding at least nbytes, or None."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {nbytes}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(func: str, status: int):
    if status != SBL_OK:
        raise SblError(func, status)


# ---------------------------------------------------------------- the C ABI, by name

def sbl_abi_version() -> int:
    return load().sbl_abi_version()


def sbl_packed_bytes(n_out: int, k: int, n: int, m: int, fmt: int) -> int:
    return load().sbl_packed_bytes(n_out, k, n, m, fmt)


def sbl_meta_bytes(n_out: int, k: int, fmt: int) -> int:
    return load().sbl_meta_bytes(n_out, k, fmt)


def sbl_workspace_bytes(n_out: int, k: int) -> int:
    return load().sbl_workspace_bytes(n_out, k)


def sbl_workspace_init(workspace, stream=None):
    """Zero-fill a whole workspace tensor (any dtype) with the library's kernel."""
    lib = load()
    nbytes = (workspace.numel() * workspace.element_size()) // 8 * 8
    _check("sbl_workspace_init",
           lib.sbl_workspace_init(_ptr(workspace, None, nbytes, "workspace"), nbytes, _stream(stream)))


_W16 = (torch.int16, torch.uint16, torch.bfloat16)


def sbl_quant_weights(w_bf16, n: int, m: int, beta, workspace, mask_bits=None, codes=None,
                      fmt: int = SBL_FMT_DENSE2, packed=None, meta=None, stream=None):
    """w_bf16: [n_out][k] BF16 (or its 16-bit patterns as int16/uint16)."""
    lib = load()
    n_out, k = w_bf16.shape
    pb = lib.sbl_packed_bytes(n_out, k, n, m, fmt) if packed is not None else 0
    mb = n_out * k // 8
    st = lib.sbl_quant_weights(
        _ptr(w_bf16, _W16, n_out * k * 2, "w_bf16"), n_out, k, n, m,
        _ptr(beta, torch.float32, 4, "beta"),
        _ptr(mask_bits, torch.uint8, mb, "mask_bits"),
        _ptr(codes, torch.int8, n_out * k, "codes"),
        fmt, _ptr(packed, torch.uint8, max(pb, 0), "packed"),
        _ptr(meta, torch.uint8, mb, "meta") if fmt == SBL_FMT_NM else None,
        _ptr(workspace, None, lib.sbl_workspace_bytes(n_out, k), "workspace"),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream))
    _check("sbl_quant_weights", st)


def _nbytes(t):
    return t.numel() * t.element_size() if t is not None else 0


def _quant_items(lib, items, n: int, m: int, fmt: int, workspaces: bool = True):
    arr = (QuantItem * len(items))()
    for i, it in enumerate(items):
        w = it["w"]
        n_out, k = w.shape
        packed = it.get("packed")
        pb = lib.sbl_packed_bytes(n_out, k, n, m, fmt) if packed is not None else 0
        mb = n_out * k // 8
        ws = it["workspace"] if workspaces else None
        arr[i] = QuantItem(
            _ptr(w, _W16, n_out * k * 2, "w"), n_out, k, _ptr(it["beta"], torch.float32, 4, "beta"),
            _ptr(it.get("mask_bits"), torch.uint8, mb, "mask_bits"),
            _ptr(it.get("codes"), torch.int8, n_out * k, "codes"),
            _ptr(packed, torch.uint8, max(pb, 0), "packed"),
            _ptr(it.get("meta"), torch.uint8, mb, "meta") if fmt == SBL_FMT_NM else None,
            _ptr(ws, None, lib.sbl_workspace_bytes(n_out, k), "workspace") if workspaces else None,
            _nbytes(ws))
    return arr


def sbl_quant_weights_batch(items, n: int, m: int, fmt: int = SBL_FMT_DENSE2, stream=None, flags: int = 0):
    """items: sequence of dicts with keys w (BF16 [n_out][k]), beta, workspace and the
    optional outputs mask_bits, codes, packed, meta (as in sbl_quant_weights)."""
    lib = load()
    arr = _quant_items(lib, items, n, m, fmt)
    if flags:
        _check("sbl_quant_weights_batch_ex",
               lib.sbl_quant_weights_batch_ex(arr, len(items), n, m, fmt, flags, _stream(stream)))
    else:
        _check("sbl_quant_weights_batch",
               lib.sbl_quant_weights_batch(arr, len(items), n, m, fmt, _stream(stream)))


def sbl_quant_weights_batch_noalloc(items, n: int, m: int, fmt: int = SBL_FMT_DENSE2, stream=None):
    """sbl_quant_weights_batch without caller workspaces: the library's fixed
    per-GPU scratch array serves every item (a "workspace" key is ignored)."""
    lib = load()
    arr = _quant_items(lib, items, n, m, fmt, workspaces=False)
    _check("sbl_quant_weights_batch_noalloc",
           lib.sbl_quant_weights_batch_noalloc(arr, len(items), n, m, fmt, _stream(stream)))


def sbl_pack(codes, mask_bits, n: int, m: int, fmt: int, packed, meta=None, stream=None):
    lib = load()
    n_out, k = codes.shape
    pb = lib.sbl_packed_bytes(n_out, k, n, m, fmt)
    mb = n_out * k // 8
    st = lib.sbl_pack(_ptr(codes, torch.int8, n_out * k, "codes"),
                      _ptr(mask_bits, torch.uint8, mb, "mask_bits") if fmt == SBL_FMT_NM else None,
                      n_out, k, n, m, fmt, _ptr(packed, torch.uint8, max(pb, 0), "packed"),
                      _ptr(meta, torch.uint8, mb, "meta") if fmt == SBL_FMT_NM else None,
                      _stream(stream))
    _check("sbl_pack", st)


def sbl_quant_acts(x, xq, gamma, stream=None):
    lib = load()
    m_tok, k = x.shape
    st = lib.sbl_quant_acts(_ptr(x, torch.float32, m_tok * k * 4, "x"), m_tok, k,
                            _ptr(xq, torch.int8, m_tok * k, "xq"),
                            _ptr(gamma, torch.float32, m_tok * 4, "gamma"), _stream(stream))
    _check("sbl_quant_acts", st)


def sbl_linear(packed, meta, fmt: int, n: int, m: int, beta, xq, gamma, n_out: int, y, acc=None,
               stream=None):
    lib = load()
    m_tok, k = xq.shape
    pb = lib.sbl_packed_bytes(n_out, k, n, m, fmt) if n_out > 0 else 0
    mb = n_out * k // 8
    st = lib.sbl_linear(_ptr(packed, torch.uint8, max(pb, 0), "packed"),
                        _ptr(meta, torch.uint8, mb, "meta") if fmt == SBL_FMT_NM else None,
                        fmt, n, m, _ptr(beta, torch.float32, 4, "beta"),
                        _ptr(xq, torch.int8, m_tok * k, "xq"),
                        _ptr(gamma, torch.float32, m_tok * 4, "gamma"), m_tok, n_out, k,
                        _ptr(y, torch.float32, m_tok * n_out * 4, "y"),
                        _ptr(acc, torch.int32, m_tok * n_out * 4, "acc"), _stream(stream))
    _check("sbl_linear", st)


def sbl_workspace_bytes_grouped(n_out: int, k: int, rows_per_group: int) -> int:
    return load().sbl_workspace_bytes_grouped(n_out, k, rows_per_group)


def sbl_quant_weights_grouped(w_bf16, n: int, m: int, rows_per_group: int, beta, workspace, mask_bits=None,
                              codes=None, fmt: int = SBL_FMT_DENSE2, packed=None, meta=None, stream=None):
    """Group scales: beta fp32 [ceil(n_out / rows_per_group)], one per block of output rows."""
    lib = load()
    n_out, k = w_bf16.shape
    groups = -(-n_out // rows_per_group) if rows_per_group > 0 else 1
    pb = lib.sbl_packed_bytes(n_out, k, n, m, fmt) if packed is not None else 0
    st = lib.sbl_quant_weights_grouped(
        _ptr(w_bf16, _W16, n_out * k * 2, "w_bf16"), n_out, k, n, m, rows_per_group,
        _ptr(beta, torch.float32, 4 * groups, "beta"),
        _ptr(mask_bits, torch.uint8, n_out * k // 8, "mask_bits"), _ptr(codes, torch.int8, n_out * k, "codes"),
        fmt, _ptr(packed, torch.uint8, max(pb, 0), "packed"),
        _ptr(meta, torch.uint8, n_out * k // 8, "meta") if fmt == SBL_FMT_NM else None,
        _ptr(workspace, None, max(lib.sbl_workspace_bytes_grouped(n_out, k, rows_per_group), 0), "workspace"),
        _nbytes(workspace), _stream(stream))
    _check("sbl_quant_weights_grouped", st)


def sbl_linear_grouped(packed, meta, fmt: int, n: int, m: int, beta, rows_per_group: int, xq, gamma, n_out: int, y,
                       acc=None, stream=None):
    lib = load()
    m_tok, k = xq.shape
    groups = -(-n_out // rows_per_group) if rows_per_group > 0 else 1
    pb = lib.sbl_packed_bytes(n_out, k, n, m, fmt) if n_out > 0 else 0
    st = lib.sbl_linear_grouped(_ptr(packed, torch.uint8, max(pb, 0), "packed"),
                                _ptr(meta, torch.uint8, n_out * k // 8, "meta") if fmt == SBL_FMT_NM else None,
                                fmt, n, m, _ptr(beta, torch.float32, 4 * groups, "beta"), rows_per_group,
                                _ptr(xq, torch.int8, m_tok * k, "xq"), _ptr(gamma, torch.float32, m_tok * 4, "gamma"),
                                m_tok, n_out, k, _ptr(y, torch.float32, m_tok * n_out * 4, "y"),
                                _ptr(acc, torch.int32, m_tok * n_out * 4, "acc"), _stream(stream))
    _check("sbl_linear_grouped", st)


def sbl_workspace_bytes_blocked(n_out: int, k: int, rows_per_group: int, cols_per_group: int) -> int:
    return load().sbl_workspace_bytes_blocked(n_out, k, rows_per_group, cols_per_group)


def sbl_quant_weights_blocked(w_bf16, n: int, m: int, rows_per_group: int, cols_per_group: int, beta, workspace,
                              mask_bits=None, codes=None, fmt: int = SBL_FMT_DENSE2, packed=None, meta=None,
                              stream=None):
    """Block scales: beta fp32 [ceil(n_out / rows_per_group)][k // cols_per_group]."""
    lib = load()
    n_out, k = w_bf16.shape
    gr = -(-n_out // rows_per_group) if rows_per_group > 0 else 1
    gk = k // cols_per_group if cols_per_group > 0 else 1
    pb = lib.sbl_packed_bytes(n_out, k, n, m, fmt) if packed is not None else 0
    wsb = lib.sbl_workspace_bytes_blocked(n_out, k, rows_per_group, cols_per_group)
    st = lib.sbl_quant_weights_blocked(
        _ptr(w_bf16, _W16, n_out * k * 2, "w_bf16"), n_out, k, n, m, rows_per_group, cols_per_group,
        _ptr(beta, torch.float32, 4 * gr * gk, "beta"),
        _ptr(mask_bits, torch.uint8, n_out * k // 8, "mask_bits"), _ptr(codes, torch.int8, n_out * k, "codes"),
        fmt, _ptr(packed, torch.uint8, max(pb, 0), "packed"),
        _ptr(meta, torch.uint8, n_out * k // 8, "meta") if fmt == SBL_FMT_NM else None,
        _ptr(workspace, None, max(wsb, 0), "workspace"), _nbytes(workspace), _stream(stream))
    _check("sbl_quant_weights_blocked", st)


def sbl_linear_blocked(packed, meta, fmt: int, n: int, m: int, beta, rows_per_group: int, xq, gamma, kg: int,
                       n_out: int, y, stream=None):
    """Products with block scales: beta [ceil(n_out / rows_per_group)][k // kg]."""
    lib = load()
    m_tok, k = xq.shape
    gr = -(-n_out // rows_per_group) if rows_per_group > 0 else 1
    gk = k // kg if kg > 0 else 1
    pb = lib.sbl_packed_bytes(n_out, k, n, m, fmt) if n_out > 0 else 0
    st = lib.sbl_linear_blocked(_ptr(packed, torch.uint8, max(pb, 0), "packed"),
                                _ptr(meta, torch.uint8, n_out * k // 8, "meta") if fmt == SBL_FMT_NM else None,
                                fmt, n, m, _ptr(beta, torch.float32, 4 * gr * gk, "beta"), rows_per_group,
                                _ptr(xq, torch.int8, m_tok * k, "xq"),
                                _ptr(gamma, torch.float32, m_tok * gk * 4, "gamma"), kg, m_tok, n_out, k,
                                _ptr(y, torch.float32, m_tok * n_out * 4, "y"), _stream(stream))
    _check("sbl_linear_blocked", st)


def sbl_quant_acts_kgrouped(x, kg: int, xq, gamma, stream=None):
    """x fp32 [m_tok][k] -> xq int8 [m_tok][k], gamma fp32 [m_tok][k // kg]."""
    lib = load()
    m_tok, k = x.shape
    st = lib.sbl_quant_acts_kgrouped(_ptr(x, torch.float32, m_tok * k * 4, "x"), m_tok, k, kg,
                                     _ptr(xq, torch.int8, m_tok * k, "xq"),
                                     _ptr(gamma, torch.float32, m_tok * (k // kg) * 4, "gamma"), _stream(stream))
    _check("sbl_quant_acts_kgrouped", st)


def sbl_linear_kgrouped(packed, meta, fmt: int, n: int, m: int, beta, rows_per_group: int, xq, gamma, kg: int,
                        n_out: int, y, stream=None):
    lib = load()
    m_tok, k = xq.shape
    groups = -(-n_out // rows_per_group) if rows_per_group > 0 else 1
    pb = lib.sbl_packed_bytes(n_out, k, n, m, fmt) if n_out > 0 else 0
    st = lib.sbl_linear_kgrouped(_ptr(packed, torch.uint8, max(pb, 0), "packed"),
                                 _ptr(meta, torch.uint8, n_out * k // 8, "meta") if fmt == SBL_FMT_NM else None,
                                 fmt, n, m, _ptr(beta, torch.float32, 4 * groups, "beta"), rows_per_group,
                                 _ptr(xq, torch.int8, m_tok * k, "xq"),
                                 _ptr(gamma, torch.float32, m_tok * (k // kg) * 4, "gamma"), kg, m_tok, n_out, k,
                                 _ptr(y, torch.float32, m_tok * n_out * 4, "y"), _stream(stream))
    _check("sbl_linear_kgrouped", st)


def sbl_backward_workspace_bytes(m_tok: int, n_out: int, k: int) -> int:
    return load().sbl_backward_workspace_bytes(m_tok, n_out, k)


def new_backward_workspace(m_tok: int, n_out: int, k: int, device="cuda"):
    """Scratch for sbl_linear_backward(..., workspace=) at these sizes (any contents)."""
    nbytes = sbl_backward_workspace_bytes(m_tok, n_out, k)
    if nbytes < 0:
        raise ValueError("unsupported shape")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def sbl_linear_backward(dy, packed, meta, fmt: int, n: int, m: int, beta, x, xq, gamma, dx=None, dw=None,
                        workspace=None, stream=None):
    """Backward of the layer (dual straight-through estimator): dy BF16 [m_tok][n_out];
    dx fp32 [m_tok][k] and/or dw fp32 [n_out][k] outputs (either may be None).  With a
    workspace (uint8, sbl_backward_workspace_bytes(m_tok, n_out, k) bytes) the call goes
    to sbl_linear_backward_ws."""
    lib = load()
    m_tok, n_out = dy.shape
    k = (xq if xq is not None else x).shape[1]
    pb = lib.sbl_packed_bytes(n_out, k, n, m, fmt) if dx is not None else 0
    if workspace is not None:
        wsb = workspace.numel() * workspace.element_size()
        fn, extra, name = lib.sbl_linear_backward_ws, (_ptr(workspace, None, wsb, "workspace"), wsb), \
            "sbl_linear_backward_ws"
    else:
        fn, extra, name = lib.sbl_linear_backward, (), "sbl_linear_backward"
    st = fn(
        _ptr(dy, _W16, m_tok * n_out * 2, "dy"), m_tok, n_out, k,
        _ptr(packed, torch.uint8, max(pb, 0), "packed") if dx is not None else None,
        _ptr(meta, torch.uint8, n_out * k // 8, "meta") if dx is not None and fmt == SBL_FMT_NM else None,
        fmt, n, m,
        _ptr(beta, torch.float32, 4, "beta") if dx is not None else None,
        _ptr(x, torch.float32, m_tok * k * 4, "x") if dx is not None else None,
        _ptr(xq, torch.int8, m_tok * k, "xq") if dw is not None else None,
        _ptr(gamma, torch.float32, m_tok * 4, "gamma"),
        _ptr(dx, torch.float32, m_tok * k * 4, "dx"), _ptr(dw, torch.float32, n_out * k * 4, "dw"),
        *extra, _stream(stream))
    _check(name, st)


def sbl_linear_batch(items, fmt: int, n: int, m: int, stream=None):
    """items: sequence of dicts with keys packed, meta, beta, xq, gamma, n_out, y[, acc]."""
    lib = load()
    arr = (LinearItem * len(items))()
    for i, it in enumerate(items):
        m_tok, k = it["xq"].shape
        n_out = it["n_out"]
        pb = lib.sbl_packed_bytes(n_out, k, n, m, fmt) if n_out > 0 else 0
        arr[i] = LinearItem(
            _ptr(it["packed"], torch.uint8, max(pb, 0), "packed"),
            _ptr(it.get("meta"), torch.uint8, n_out * k // 8, "meta") if fmt == SBL_FMT_NM else None,
            _ptr(it["beta"], torch.float32, 4, "beta"), _ptr(it["xq"], torch.int8, m_tok * k, "xq"),
            _ptr(it["gamma"], torch.float32, m_tok * 4, "gamma"), m_tok, n_out, k,
            _ptr(it["y"], torch.float32, m_tok * n_out * 4, "y"),
            _ptr(it.get("acc"), torch.int32, m_tok * n_out * 4, "acc"))
    _check("sbl_linear_batch", lib.sbl_linear_batch(arr, len(items), fmt, n, m, _stream(stream)))


def sbl_linear_acts_batch(x, xq, gamma, items, fmt: int, n: int, m: int, stream=None):
    """x: [m_tok][k] fp32 input; xq, gamma: its quantized form (outputs);
    items: sequence of dicts with keys packed, meta, beta, n_out, y[, acc]."""
    lib = load()
    m_tok, k = x.shape
    arr = (LinearItem * len(items))()
    for i, it in enumerate(items):
        n_out = it["n_out"]
        pb = lib.sbl_packed_bytes(n_out, k, n, m, fmt) if n_out > 0 else 0
        arr[i] = LinearItem(
            _ptr(it["packed"], torch.uint8, max(pb, 0), "packed"),
            _ptr(it.get("meta"), torch.uint8, n_out * k // 8, "meta") if fmt == SBL_FMT_NM else None,
            _ptr(it["beta"], torch.float32, 4, "beta"), None, None, m_tok, n_out, k,
            _ptr(it["y"], torch.float32, m_tok * n_out * 4, "y"),
            _ptr(it.get("acc"), torch.int32, m_tok * n_out * 4, "acc"))
    st = lib.sbl_linear_acts_batch(_ptr(x, torch.float32, m_tok * k * 4, "x"), m_tok, k,
                                   _ptr(xq, torch.int8, m_tok * k, "xq"),
                                   _ptr(gamma, torch.float32, m_tok * 4, "gamma"), arr, len(items), fmt, n, m,
                                   _stream(stream))
    _check("sbl_linear_acts_batch", st)


# ---------------------------------------------------------------- allocating conveniences

def new_workspace(n_out: int, k: int, device="cuda"):
    """A workspace for n_out x k matrices (reusable, call after call; any contents)."""
    nbytes = sbl_workspace_bytes(n_out, k)
    if nbytes < 0:
        raise ValueError("unsupported shape")
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def quant_weights(w_bf16, n: int, m: int, fmt: int = SBL_FMT_DENSE2, want_codes: bool = False,
                  workspace=None, stream=None):
    """Allocate outputs and run sbl_quant_weights; returns a dict of device tensors."""
    n_out, k = w_bf16.shape
    dev = w_bf16.device
    out = {"beta": torch.empty(1, dtype=torch.float32, device=dev),
           "mask": torch.empty((n_out, k // 8), dtype=torch.uint8, device=dev)}
    pb = sbl_packed_bytes(n_out, k, n, m, fmt)
    if pb < 0:
        raise ValueError("unsupported shape or pattern")
    out["packed"] = torch.empty(pb, dtype=torch.uint8, device=dev)
    out["meta"] = torch.empty((n_out, k // 8), dtype=torch.uint8, device=dev) if fmt == SBL_FMT_NM else None
    out["codes"] = torch.empty((n_out, k), dtype=torch.int8, device=dev) if want_codes else None
    ws = workspace if workspace is not None else new_workspace(n_out, k, dev)
    sbl_quant_weights(w_bf16, n, m, out["beta"], ws, mask_bits=out["mask"], codes=out["codes"],
                      fmt=fmt, packed=out["packed"], meta=out["meta"], stream=stream)
    return out


def quant_acts(x, stream=None):
    m_tok, k = x.shape
    xq = torch.empty((m_tok, k), dtype=torch.int8, device=x.device)
    gamma = torch.empty(m_tok, dtype=torch.float32, device=x.device)
    sbl_quant_acts(x, xq, gamma, stream=stream)
    return xq, gamma


def linear(packed, meta, fmt, n, m, beta, xq, gamma, n_out, want_acc=False, stream=None):
    m_tok = xq.shape[0]
    y = torch.empty((m_tok, n_out), dtype=torch.float32, device=xq.device)
    acc = torch.empty((m_tok, n_out), dtype=torch.int32, device=xq.device) if want_acc else None
    sbl_linear(packed, meta, fmt, n, m, beta, xq, gamma, n_out, y, acc, stream=stream)
    return y, acc
