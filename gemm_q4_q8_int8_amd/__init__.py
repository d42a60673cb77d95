"""Python binding of liblq (block-quantized GEMV / GEMM for MI355X).

Argument marshalling only: every function here has the name of the C entry
point it calls (see include/lq.h), turns torch tensors into device pointers
and sizes, passes torch's current HIP stream, and raises LQError when the
library returns a failure status.  All arithmetic runs in the HIP kernels of
liblq.so; there is no fallback path.  If liblq.so has not been built, every
call raises LibraryNotBuilt.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblq.so")

LQ_Q4_0, LQ_Q8_0, LQ_I8B64, LQ_I8B32 = 0, 1, 2, 3
LQ_F32, LQ_F16, LQ_BF16 = 0, 1, 2
FORMATS = {"q4_0": LQ_Q4_0, "q8_0": LQ_Q8_0, "i8b64": LQ_I8B64, "i8b32": LQ_I8B32}

# Every symbol include/lq.h declares.
EXPORTS = ("lq_abi_version", "lq_init", "lq_block_elems", "lq_packed_bytes", "lq_scale_offset",
           "lq_gguf_bytes", "lq_repack_gguf", "lq_pack_planes", "lq_quantize", "lq_dequant_f32",
           "lq_dequant_f16", "lq_gemv_workspace_bytes", "lq_gemv", "lq_gemv_batch",
           "lq_gemv_batch_noalloc", "lq_gemv_multi",
           "lq_gemv_multi_batch", "lq_quantize_act", "lq_gemv_q8act", "lq_gemm_workspace_bytes",
           "lq_gemm", "lq_gemm_batch",
           "lq_matmul", "lq_status_str", "lq_last_error")


class LibraryNotBuilt(RuntimeError):
    pass


class LQError(RuntimeError):
    def __init__(self, status: int, name: str, message: str):
        super().__init__(f"{name}: {message}")
        self.status = status
        self.name = name
        self.message = message


class lq_gemv_desc(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("xdt", ctypes.c_int32), ("W", ctypes.c_void_p),
                ("x", ctypes.c_void_p), ("y", ctypes.c_void_p), ("N", ctypes.c_int64),
                ("K", ctypes.c_int64)]


class lq_gemv_multi_desc(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("xdt", ctypes.c_int32), ("W", ctypes.c_void_p),
                ("X", ctypes.c_void_p), ("Y", ctypes.c_void_p), ("M", ctypes.c_int64),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class lq_gemm_desc(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("Y", ctypes.c_void_p), ("N", ctypes.c_int64)]


LQ_GEMM_MAX_GROUP = 4

_lib = None


def load(path: str = LIB_PATH):
    """Load liblq.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise LibraryNotBuilt(f"{path} is missing: build it with gemm_q4_q8_int8_amd.build.build()")
    L = ctypes.CDLL(path)
    i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    sig = {
        "lq_abi_version": ([], i32),
        "lq_init": ([], i32),
        "lq_block_elems": ([i32], i32),
        "lq_packed_bytes": ([i32, i64, i64], sz),
        "lq_scale_offset": ([i32, i64, i64], sz),
        "lq_gguf_bytes": ([i32, i64, i64], sz),
        "lq_repack_gguf": ([i32, vp, vp, i64, i64, vp], i32),
        "lq_pack_planes": ([i32, vp, vp, vp, i64, i64, vp], i32),
        "lq_quantize": ([i32, vp, i32, vp, i64, i64, vp], i32),
        "lq_dequant_f32": ([i32, vp, vp, i64, i64, vp], i32),
        "lq_dequant_f16": ([i32, vp, vp, i64, i64, vp], i32),
        "lq_gemv_workspace_bytes": ([], sz),
        "lq_gemv": ([i32, vp, vp, i32, vp, i64, i64, vp, sz, vp], i32),
        "lq_gemv_batch": ([ctypes.POINTER(lq_gemv_desc), i32, vp, sz, vp], i32),
        "lq_gemv_batch_noalloc": ([ctypes.POINTER(lq_gemv_desc), i32, vp], i32),
        "lq_gemv_multi": ([i32, vp, vp, i32, vp, i64, i64, i64, vp, sz, vp], i32),
        "lq_gemv_multi_batch": ([ctypes.POINTER(lq_gemv_multi_desc), i32, vp, sz, vp], i32),
        "lq_quantize_act": ([vp, i32, i64, i64, vp, vp, vp, vp], i32),
        "lq_gemv_q8act": ([i32, vp, vp, vp, vp, vp, i64, i64, i64, vp, sz, vp], i32),
        "lq_gemm_workspace_bytes": ([i32, i64, i64, i64], sz),
        "lq_gemm": ([i32, vp, vp, i32, vp, i64, i64, i64, vp, sz, vp], i32),
        "lq_gemm_batch": ([i32, vp, i32, i64, i64, ctypes.POINTER(lq_gemm_desc), i32, vp, sz, vp], i32),
        "lq_matmul": ([i32, vp, vp, i32, vp, i64, i64, i64, vp, sz, vp], i32),
        "lq_status_str": ([i32], ctypes.c_char_p),
        "lq_last_error": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        L = load()
        raise LQError(status, L.lq_status_str(status).decode(), L.lq_last_error().decode())


def _ptr(t):
    """Device pointer of a tensor (or a raw integer address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _ws_bytes(ws, ws_bytes):
    """Workspace size: as given, else the whole tensor (0 without one)."""
    if ws_bytes is not None:
        return int(ws_bytes)
    if ws is None or isinstance(ws, int):
        return 0
    return ws.numel() * ws.element_size()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _xdt(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return LQ_F32
    if t.dtype == torch.float16:
        return LQ_F16
    raise TypeError(f"activations must be float32 or float16, got {t.dtype}")


def _fmt(fmt) -> int:
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


# ------------------------------------------------------------------ queries

def lq_abi_version() -> int:
    return load().lq_abi_version()


def lq_init():
    _check(load().lq_init())


def lq_block_elems(fmt) -> int:
    return load().lq_block_elems(_fmt(fmt))


def lq_packed_bytes(fmt, N, K) -> int:
    return load().lq_packed_bytes(_fmt(fmt), N, K)


def lq_scale_offset(fmt, N, K) -> int:
    return load().lq_scale_offset(_fmt(fmt), N, K)


def lq_gguf_bytes(fmt, N, K) -> int:
    return load().lq_gguf_bytes(_fmt(fmt), N, K)


def lq_gemv_workspace_bytes() -> int:
    return load().lq_gemv_workspace_bytes()


def lq_gemm_workspace_bytes(fmt, M, N, K) -> int:
    return load().lq_gemm_workspace_bytes(_fmt(fmt), M, N, K)


def lq_status_str(status: int) -> str:
    return load().lq_status_str(status).decode()


def lq_last_error() -> str:
    return load().lq_last_error().decode()


# -------------------------------------------------------------- operations

def lq_repack_gguf(fmt, src, dst, N, K, stream=None):
    _check(load().lq_repack_gguf(_fmt(fmt), _ptr(src), _ptr(dst), N, K, _stream(stream)))


def lq_pack_planes(fmt, codes, scales, dst, N, K, stream=None):
    _check(load().lq_pack_planes(_fmt(fmt), _ptr(codes), _ptr(scales), _ptr(dst), N, K,
                                 _stream(stream)))


def lq_quantize(fmt, src, W, N, K, stream=None, sdt=None):
    """src: float32 / float16 / bfloat16 tensor (N x K row-major)."""
    if sdt is None:
        import torch
        sdt = LQ_BF16 if src.dtype == torch.bfloat16 else _xdt(src)
    _check(load().lq_quantize(_fmt(fmt), _ptr(src), sdt, _ptr(W), N, K, _stream(stream)))


def lq_dequant_f32(fmt, W, out, N, K, stream=None):
    _check(load().lq_dequant_f32(_fmt(fmt), _ptr(W), _ptr(out), N, K, _stream(stream)))


def lq_dequant_f16(fmt, W, out, N, K, stream=None):
    _check(load().lq_dequant_f16(_fmt(fmt), _ptr(W), _ptr(out), N, K, _stream(stream)))


def lq_gemv(fmt, W, x, y, N, K, ws=None, ws_bytes=None, stream=None, xdt=None):
    """ws: optional GEMV workspace (lq_gemv_workspace_bytes() bytes)."""
    xdt = _xdt(x) if xdt is None else xdt
    _check(load().lq_gemv(_fmt(fmt), _ptr(W), _ptr(x), xdt, _ptr(y), N, K, _ptr(ws),
                          _ws_bytes(ws, ws_bytes), _stream(stream)))


def lq_gemv_batch(descs, ws=None, ws_bytes=None, stream=None):
    """descs: sequence of (fmt, W, x, y, N, K) tuples of tensors / sizes."""
    arr = (lq_gemv_desc * max(1, len(descs)))()
    for i, (fmt, W, x, y, N, K) in enumerate(descs):
        arr[i] = lq_gemv_desc(_fmt(fmt), _xdt(x), _ptr(W), _ptr(x), _ptr(y), N, K)
    _check(load().lq_gemv_batch(arr, len(descs), _ptr(ws), _ws_bytes(ws, ws_bytes), _stream(stream)))


def lq_gemv_batch_noalloc(descs, stream=None):
    """lq_gemv_batch with the library's static workspace (allocates nothing)."""
    arr = (lq_gemv_desc * max(1, len(descs)))()
    for i, (fmt, W, x, y, N, K) in enumerate(descs):
        arr[i] = lq_gemv_desc(_fmt(fmt), _xdt(x), _ptr(W), _ptr(x), _ptr(y), N, K)
    _check(load().lq_gemv_batch_noalloc(arr, len(descs), _stream(stream)))


def lq_gemv_multi(fmt, W, X, Y, M, N, K, ws=None, ws_bytes=None, stream=None, xdt=None):
    xdt = _xdt(X) if xdt is None else xdt
    _check(load().lq_gemv_multi(_fmt(fmt), _ptr(W), _ptr(X), xdt, _ptr(Y), M, N, K, _ptr(ws),
                                _ws_bytes(ws, ws_bytes), _stream(stream)))


def lq_gemv_multi_batch(descs, ws=None, ws_bytes=None, stream=None):
    """descs: sequence of (fmt, W, X, Y, M, N, K) tuples of tensors / sizes."""
    arr = (lq_gemv_multi_desc * max(1, len(descs)))()
    for i, (fmt, W, X, Y, M, N, K) in enumerate(descs):
        arr[i] = lq_gemv_multi_desc(_fmt(fmt), _xdt(X), _ptr(W), _ptr(X), _ptr(Y), M, N, K)
    _check(load().lq_gemv_multi_batch(arr, len(descs), _ptr(ws), _ws_bytes(ws, ws_bytes),
                                      _stream(stream)))


def lq_quantize_act(X, M, K, q, s, sum, stream=None, xdt=None):
    """X: float32 / float16 (M x K); q: int8 (M x K); s: float32 and sum: int32 (M x K/32)."""
    xdt = _xdt(X) if xdt is None else xdt
    _check(load().lq_quantize_act(_ptr(X), xdt, M, K, _ptr(q), _ptr(s), _ptr(sum), _stream(stream)))


def lq_gemv_q8act(fmt, W, q, s, sum, Y, M, N, K, ws=None, ws_bytes=None, stream=None):
    _check(load().lq_gemv_q8act(_fmt(fmt), _ptr(W), _ptr(q), _ptr(s), _ptr(sum), _ptr(Y), M, N, K, _ptr(ws),
                                _ws_bytes(ws, ws_bytes), _stream(stream)))


def lq_gemm(fmt, W, X, Y, M, N, K, ws=None, ws_bytes=None, stream=None, xdt=None):
    xdt = _xdt(X) if xdt is None else xdt
    _check(load().lq_gemm(_fmt(fmt), _ptr(W), _ptr(X), xdt, _ptr(Y), M, N, K, _ptr(ws),
                          _ws_bytes(ws, ws_bytes), _stream(stream)))


def lq_gemm_batch(fmt, X, M, K, descs, ws=None, ws_bytes=None, stream=None, xdt=None):
    """descs: sequence of (W, Y, N): weight matrices sharing X, M and K."""
    xdt = _xdt(X) if xdt is None else xdt
    arr = (lq_gemm_desc * max(1, len(descs)))()
    for i, (W, Y, N) in enumerate(descs):
        arr[i] = lq_gemm_desc(_ptr(W), _ptr(Y), N)
    _check(load().lq_gemm_batch(_fmt(fmt), _ptr(X), xdt, M, K, arr, len(descs), _ptr(ws),
                                _ws_bytes(ws, ws_bytes), _stream(stream)))


def lq_matmul(fmt, W, X, Y, M, N, K, ws=None, ws_bytes=None, stream=None, xdt=None):
    xdt = _xdt(X) if xdt is None else xdt
    _check(load().lq_matmul(_fmt(fmt), _ptr(W), _ptr(X), xdt, _ptr(Y), M, N, K, _ptr(ws),
                            _ws_bytes(ws, ws_bytes), _stream(stream)))
