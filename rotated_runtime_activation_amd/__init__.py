"""Python binding of librrs, the gfx950 Rotated Runtime Smooth A4W4 linear.

Argument marshalling only: every function below checks tensor dtypes,
shapes, devices and contiguity, takes raw device pointers and the current
HIP stream, and calls the C entry point of the same name declared in
``include/rrs.h``. All arithmetic runs in the HIP kernels of librrs; there is
no fallback. If the library has not been built the import still succeeds but
every call raises ``RRSLibraryMissing``.
"""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "librrs.so")

RRS_OK, RRS_EINVAL, RRS_EUNSUPPORTED, RRS_EHIP, RRS_ETOOBIG = 0, -1, -2, -3, -4
RRS_NOALLOC_SCRATCH_BYTES = 24 << 20
RRS_FLAG_NO_ROTATE = 1
RRS_FLAG_NO_SMOOTH = 2
RRS_FLAG_TWO_PASS = 4
RRS_FLAG_TEST_GIVE_UP = 8

# every symbol include/rrs.h declares
EXPORTS = (
    "rrs_status_string", "rrs_version", "rrs_weight_bytes", "rrs_workspace_bytes",
    "rrs_sync_bytes", "rrs_workspace_init", "rrs_calibrate_workspace_bytes",
    "rrs_calibrate_perm", "rrs_prepare_weights", "rrs_linear", "rrs_frontend", "rrs_gemm",
    "rrs_gemm_partials", "rrs_frontend_passes", "rrs_gemm_form",
    "rrs_calibrate_perm_signed", "rrs_prepare_weights_signed", "rrs_linear_signed",
    "rrs_frontend_signed", "rrs_calibrate_perm_ex", "rrs_prepare_weights_ex", "rrs_linear_ex",
    "rrs_linear_noalloc", "rrs_codes_bytes",
)


class RRSLibraryMissing(RuntimeError):
    pass


class RRSError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


_lib = None


def _declare(lib):
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    sig = {
        "rrs_status_string": (ctypes.c_char_p, [i]),
        "rrs_version": (ctypes.c_char_p, []),
        "rrs_weight_bytes": (sz, [i, i]),
        "rrs_codes_bytes": (sz, [i, i]),
        "rrs_workspace_bytes": (sz, [i, i, i]),
        "rrs_sync_bytes": (sz, [i, i]),
        "rrs_workspace_init": (i, [vp, sz, vp]),
        "rrs_calibrate_workspace_bytes": (sz, [i]),
        "rrs_calibrate_perm": (i, [vp, i, i, vp, vp, sz, vp]),
        "rrs_prepare_weights": (i, [vp, i, i, vp, vp, vp]),
        "rrs_linear": (i, [vp, i, i, i, i, vp, vp, vp, vp, sz, vp]),
        "rrs_frontend": (i, [vp, i, i, i, vp, vp, vp, vp, vp, sz, i, vp]),
        "rrs_gemm": (i, [vp, vp, vp, i, i, i, i, vp, vp, vp]),
        "rrs_gemm_partials": (i, [vp, i, i, i, i, vp, i, i, i, i, vp, vp]),
        "rrs_frontend_passes": (i, [i, i, i]),
        "rrs_gemm_form": (i, [i, i, i, i]),
        "rrs_calibrate_perm_signed": (i, [vp, i, i, vp, vp, vp, sz, vp]),
        "rrs_prepare_weights_signed": (i, [vp, i, i, vp, vp, vp, vp]),
        "rrs_linear_signed": (i, [vp, i, i, i, i, vp, vp, vp, vp, vp, sz, vp]),
        "rrs_frontend_signed": (i, [vp, i, i, i, vp, vp, vp, vp, vp, vp, sz, i, vp]),
        "rrs_calibrate_perm_ex": (i, [vp, i, i, vp, i, vp, vp, sz, vp]),
        "rrs_prepare_weights_ex": (i, [vp, i, i, vp, vp, i, vp, vp]),
        "rrs_linear_ex": (i, [vp, i, i, i, i, vp, vp, i, vp, vp, vp, sz, vp]),
        "rrs_linear_noalloc": (i, [vp, i, i, i, i, vp, vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def lib():
    """The loaded librrs (ctypes). Raises RRSLibraryMissing if not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RRSLibraryMissing(
                f"{LIB_PATH} is missing: build it with `python -m rotated_runtime_activation_amd.build`")
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def _check(fn: str, status: int) -> None:
    if status != RRS_OK:
        raise RRSError(fn, status, lib().rrs_status_string(status).decode())


# ------------------------------------------------------------ size queries
@functools.lru_cache(maxsize=256)
def rrs_weight_bytes(K: int, N: int) -> int:
    return int(lib().rrs_weight_bytes(K, N))


@functools.lru_cache(maxsize=256)
def rrs_codes_bytes(rows: int, K: int) -> int:
    """Bytes of a code matrix of `rows` rows of length K in the stored
    layout (include/rrs.h): the xq buffer of rrs_frontend for M = rows."""
    return int(lib().rrs_codes_bytes(rows, K))


def rrs_workspace_bytes(M: int, K: int, G: int) -> int:
    return int(lib().rrs_workspace_bytes(M, K, G))


def rrs_sync_bytes(K: int, G: int) -> int:
    return int(lib().rrs_sync_bytes(K, G))


def rrs_calibrate_workspace_bytes(K: int) -> int:
    return int(lib().rrs_calibrate_workspace_bytes(K))


def rrs_frontend_passes(M: int, K: int, flags: int = 0) -> int:
    """Launches (1 or 3) the front end uses for M tokens on the current device."""
    n = int(lib().rrs_frontend_passes(M, K, flags))
    if n < 0:
        _check("rrs_frontend_passes", n)
    return n


RRS_GEMM_TILED = 1
RRS_GEMM_FEW_TOKENS = 2


def rrs_gemm_form(M: int, K: int, N: int, G: int) -> int:
    """GEMM kernel rrs_gemm / rrs_linear run for (M, K, N, G): RRS_GEMM_TILED
    or RRS_GEMM_FEW_TOKENS."""
    n = int(lib().rrs_gemm_form(M, K, N, G))
    if n < 0:
        _check("rrs_gemm_form", n)
    return n


def rrs_status_string(status: int) -> str:
    return lib().rrs_status_string(status).decode()


def rrs_version() -> str:
    return lib().rrs_version().decode()


# ---------------------------------------------------------- marshalling
def _torch():
    import torch
    return torch


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev(t, dtype, name: str, shape: Optional[tuple] = None, min_numel: int = 0) -> int:
    """Device address of a checked tensor argument. The checks use the
    cheapest tensor attributes: they run on every call, and for small
    shapes the host time of a call can exceed its GPU time."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and t.shape != shape:
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if min_numel and t.nbytes < min_numel:
        raise ValueError(f"{name} holds {t.nbytes} bytes, needs {min_numel}")
    return t.data_ptr()


def _nbytes(t) -> int:
    return t.nbytes


# ----------------------------------------------------------- entry points
def rrs_workspace_init(ws, stream=None) -> None:
    _check("rrs_workspace_init", lib().rrs_workspace_init(_dev(ws, None, "ws"), _nbytes(ws), _stream(stream)))


def rrs_calibrate_perm(X_cal, perm, ws, stream=None) -> None:
    torch = _torch()
    T, K = X_cal.shape
    _check("rrs_calibrate_perm", lib().rrs_calibrate_perm(
        _dev(X_cal, torch.float16, "X_cal"), T, K, _dev(perm, torch.int32, "perm", (K,)),
        _dev(ws, None, "ws"), _nbytes(ws), _stream(stream)))


def rrs_prepare_weights(W, perm, wq, stream=None) -> None:
    torch = _torch()
    K, N = W.shape
    _check("rrs_prepare_weights", lib().rrs_prepare_weights(
        _dev(W, torch.float16, "W"), K, N, _dev(perm, torch.int32, "perm", (K,)),
        _dev(wq, torch.uint8, "wq", min_numel=rrs_weight_bytes(K, N)), _stream(stream)))


def rrs_linear(X, G: int, perm, wq, Y, ws, stream=None) -> None:
    torch = _torch()
    M, K = X.shape
    N = Y.shape[1]
    _check("rrs_linear", lib().rrs_linear(
        _dev(X, torch.float16, "X"), M, K, N, G, _dev(perm, torch.int32, "perm", (K,)),
        _dev(wq, torch.uint8, "wq", min_numel=rrs_weight_bytes(K, N)),
        _dev(Y, torch.float32, "Y", (M, N)), _dev(ws, None, "ws"), _nbytes(ws), _stream(stream)))


def rrs_frontend(X, G: int, perm, xq, dx, S, ws, flags: int = 0, stream=None) -> None:
    torch = _torch()
    M, K = X.shape
    _check("rrs_frontend", lib().rrs_frontend(
        _dev(X, torch.float16, "X"), M, K, G, _dev(perm, torch.int32, "perm", (K,)),
        _dev(xq, torch.uint8, "xq", min_numel=rrs_codes_bytes(M, K)), _dev(dx, torch.float32, "dx", (M,)),
        _dev(S, torch.float32, "S", (K // G,)), _dev(ws, None, "ws"), _nbytes(ws), flags,
        _stream(stream)))


# signed rotation X D H: dsign is int32 [K/32] holding the K-bit sign mask
# (bit j set: channel j negated)
def rrs_calibrate_perm_signed(X_cal, dsign, perm, ws, stream=None) -> None:
    torch = _torch()
    T, K = X_cal.shape
    _check("rrs_calibrate_perm_signed", lib().rrs_calibrate_perm_signed(
        _dev(X_cal, torch.float16, "X_cal"), T, K, _dev(dsign, torch.int32, "dsign", (K // 32,)),
        _dev(perm, torch.int32, "perm", (K,)), _dev(ws, None, "ws"), _nbytes(ws), _stream(stream)))


def rrs_prepare_weights_signed(W, perm, dsign, wq, stream=None) -> None:
    torch = _torch()
    K, N = W.shape
    _check("rrs_prepare_weights_signed", lib().rrs_prepare_weights_signed(
        _dev(W, torch.float16, "W"), K, N, _dev(perm, torch.int32, "perm", (K,)),
        _dev(dsign, torch.int32, "dsign", (K // 32,)),
        _dev(wq, torch.uint8, "wq", min_numel=rrs_weight_bytes(K, N)), _stream(stream)))


def rrs_linear_signed(X, G: int, perm, dsign, wq, Y, ws, stream=None) -> None:
    torch = _torch()
    M, K = X.shape
    N = Y.shape[1]
    _check("rrs_linear_signed", lib().rrs_linear_signed(
        _dev(X, torch.float16, "X"), M, K, N, G, _dev(perm, torch.int32, "perm", (K,)),
        _dev(dsign, torch.int32, "dsign", (K // 32,)),
        _dev(wq, torch.uint8, "wq", min_numel=rrs_weight_bytes(K, N)),
        _dev(Y, torch.float32, "Y", (M, N)), _dev(ws, None, "ws"), _nbytes(ws), _stream(stream)))


def rrs_frontend_signed(X, G: int, perm, dsign, xq, dx, S, ws, flags: int = 0, stream=None) -> None:
    torch = _torch()
    M, K = X.shape
    _check("rrs_frontend_signed", lib().rrs_frontend_signed(
        _dev(X, torch.float16, "X"), M, K, G, _dev(perm, torch.int32, "perm", (K,)),
        _dev(dsign, torch.int32, "dsign", (K // 32,)),
        _dev(xq, torch.uint8, "xq", min_numel=rrs_codes_bytes(M, K)), _dev(dx, torch.float32, "dx", (M,)),
        _dev(S, torch.float32, "S", (K // G,)), _dev(ws, None, "ws"), _nbytes(ws), flags,
        _stream(stream)))


# component switches (flags): dsign is None or the int32 [K/32] sign mask
def _opt_sign(dsign, K: int) -> int:
    return 0 if dsign is None else _dev(dsign, _torch().int32, "dsign", (K // 32,))


def rrs_calibrate_perm_ex(X_cal, dsign, flags: int, perm, ws, stream=None) -> None:
    torch = _torch()
    T, K = X_cal.shape
    _check("rrs_calibrate_perm_ex", lib().rrs_calibrate_perm_ex(
        _dev(X_cal, torch.float16, "X_cal"), T, K, _opt_sign(dsign, K), flags,
        _dev(perm, torch.int32, "perm", (K,)), _dev(ws, None, "ws"), _nbytes(ws), _stream(stream)))


def rrs_prepare_weights_ex(W, perm, dsign, flags: int, wq, stream=None) -> None:
    torch = _torch()
    K, N = W.shape
    _check("rrs_prepare_weights_ex", lib().rrs_prepare_weights_ex(
        _dev(W, torch.float16, "W"), K, N, _dev(perm, torch.int32, "perm", (K,)), _opt_sign(dsign, K), flags,
        _dev(wq, torch.uint8, "wq", min_numel=rrs_weight_bytes(K, N)), _stream(stream)))


def rrs_linear_ex(X, G: int, perm, dsign, flags: int, wq, Y, ws, stream=None) -> None:
    torch = _torch()
    M, K = X.shape
    N = Y.shape[1]
    _check("rrs_linear_ex", lib().rrs_linear_ex(
        _dev(X, torch.float16, "X"), M, K, N, G, _dev(perm, torch.int32, "perm", (K,)), _opt_sign(dsign, K),
        flags, _dev(wq, torch.uint8, "wq", min_numel=rrs_weight_bytes(K, N)),
        _dev(Y, torch.float32, "Y", (M, N)), _dev(ws, None, "ws"), _nbytes(ws), _stream(stream)))


def rrs_linear_noalloc(X, G: int, perm, wq, Y, stream=None) -> None:
    """rrs_linear on the library's fixed scratch (no workspace argument)."""
    torch = _torch()
    M, K = X.shape
    N = Y.shape[1]
    _check("rrs_linear_noalloc", lib().rrs_linear_noalloc(
        _dev(X, torch.float16, "X"), M, K, N, G, _dev(perm, torch.int32, "perm", (K,)),
        _dev(wq, torch.uint8, "wq", min_numel=rrs_weight_bytes(K, N)),
        _dev(Y, torch.float32, "Y", (M, N)), _stream(stream)))


def rrs_gemm(xq, dx, S, G: int, wq, Y, stream=None) -> None:
    """xq: the codes as rrs_frontend writes them (M from Y, K = G * S.numel())."""
    torch = _torch()
    M, N = Y.shape
    K = G * S.numel()
    _check("rrs_gemm", lib().rrs_gemm(
        _dev(xq, torch.uint8, "xq", min_numel=rrs_codes_bytes(M, K)), _dev(dx, torch.float32, "dx", (M,)),
        _dev(S, torch.float32, "S", (K // G,)), M, K, N, G,
        _dev(wq, torch.uint8, "wq", min_numel=rrs_weight_bytes(K, N)),
        _dev(Y, torch.float32, "Y", (M, N)), _stream(stream)))


def rrs_gemm_partials(xq, M: int, K: int, N: int, G: int, wq, m0: int, m1: int, n0: int, n1: int, P,
                      stream=None) -> None:
    torch = _torch()
    _check("rrs_gemm_partials", lib().rrs_gemm_partials(
        _dev(xq, torch.uint8, "xq", min_numel=rrs_codes_bytes(M, K)), M, K, N, G,
        _dev(wq, torch.uint8, "wq", min_numel=rrs_weight_bytes(K, N)), m0, m1, n0, n1,
        _dev(P, torch.int32, "P", (m1 - m0, n1 - n0, K // G)), _stream(stream)))


# ----------------------------------------------------------- conveniences
def codes_stored_view(buf, rows: int, K: int):
    """Writable [pairs, 2, pieces, piece bytes] view of a code matrix in the
    stored layout of include/rrs.h (row 2p + h, byte 64 c + e at [p, h, c,
    e]); `buf` is a uint8 tensor starting at the matrix."""
    kb = K // 2
    rs = (kb + 63) // 64 * 64
    pb = min(kb, 64)
    pairs = (rows + 1) // 2
    return buf.reshape(-1).as_strided((pairs, 2, kb // pb, pb), (2 * rs, 64, 128, 1))


def codes_matrix(buf, rows: int, K: int):
    """The code matrix [rows, K/2] (row-major, a copy) held in `buf` in the
    stored layout."""
    v = codes_stored_view(buf, rows, K)
    return v.reshape(v.shape[0] * 2, K // 2)[:rows]


def codes_buffer(codes, K: int, out=None):
    """A buffer holding the row-major code matrix `codes` [rows, K/2] (uint8,
    device) in the stored layout: `out` (rrs_codes_bytes(rows, K) bytes), or
    a new zeroed tensor."""
    torch = _torch()
    rows = codes.shape[0]
    if out is None:
        out = torch.zeros(rrs_codes_bytes(rows, K), dtype=torch.uint8, device=codes.device)
    v = codes_stored_view(out, rows, K)
    src = codes if rows % 2 == 0 else torch.cat([codes, torch.zeros_like(codes[:1])])
    v.copy_(src.reshape(v.shape))
    return out


def weight_views(wq, K: int, N: int):
    """(codes uint8 [N, K/2] (a copy, row-major), dw float32 [N] (a view))
    of a prepared-weight buffer (layout documented in include/rrs.h)."""
    cb = rrs_codes_bytes(N, K)
    off = (cb + 255) // 256 * 256
    return codes_matrix(wq[:cb], N, K), wq[off: off + 4 * N].view(_torch().float32)


def weight_codes_region(wq, K: int, N: int):
    """The codes region of a prepared-weight buffer (stored layout, a view)."""
    return wq[: rrs_codes_bytes(N, K)]


def workspace_codes(ws, M: int, K: int, G: int):
    """The xq region of an rrs_linear workspace (stored layout, a view), as
    rrs_gemm takes it."""
    xq_off = rrs_sync_bytes(K, G)
    return ws[xq_off: xq_off + rrs_codes_bytes(M, K)]


def workspace_regions(ws, M: int, K: int, G: int):
    """(xq region (stored layout), dx [M], S [K/G]): views into an
    rrs_linear workspace, as rrs_frontend writes and rrs_gemm reads them."""
    torch = _torch()
    a = lambda x: (x + 255) // 256 * 256
    xq_off = rrs_sync_bytes(K, G)
    dx_off = xq_off + a(rrs_codes_bytes(M, K))
    s_off = dx_off + a(4 * M)
    return (ws[xq_off: xq_off + rrs_codes_bytes(M, K)],
            ws[dx_off: dx_off + 4 * M].view(torch.float32),
            ws[s_off: s_off + 4 * (K // G)].view(torch.float32))


def workspace_views(ws, M: int, K: int, G: int):
    """(xq [M, K/2] (a row-major copy), dx [M], S [K/G] (views)) of an
    rrs_linear workspace."""
    xq, dx, S = workspace_regions(ws, M, K, G)
    return codes_matrix(xq, M, K), dx, S
