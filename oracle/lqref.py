"""ctypes wrapper of the CPU oracle ``liblqref.so`` (built from lqref.cpp).

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers; the HIP library never imports this.
The arithmetic lives in lqref.cpp; this file only moves numpy buffers across.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lqref.cpp")
_LIB = os.path.join(_HERE, "liblqref.so")

Q4_0, Q8_0, I8B64, I8B32 = 0, 1, 2, 3
F32, F16, BF16 = 0, 1, 2
FMT_NAMES = {"q4_0": Q4_0, "q8_0": Q8_0, "i8b64": I8B64, "i8b32": I8B32}
PLANAR = (I8B64, I8B32)   # int8 codes + fp32 scale plane (no GGUF form)


def build(force: bool = True) -> str:
    """Compile lqref.cpp with the host compiler (no HIP)."""
    if force or not os.path.exists(_LIB):
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread",
               "-ffp-contract=off", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _bind(L):
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    L.lqref_half_to_double.argtypes = [ctypes.c_uint16]
    L.lqref_half_to_double.restype = ctypes.c_double
    L.lqref_double_to_half.argtypes = [ctypes.c_double]
    L.lqref_double_to_half.restype = ctypes.c_uint16
    L.lqref_block_elems.argtypes = [i32]
    L.lqref_gguf_block_bytes.argtypes = [i32]
    for name in ("lqref_dequant", "lqref_dequant_f32", "lqref_dequant_f16"):
        getattr(L, name).argtypes = [i32, vp, vp, i64, i64, vp]
    L.lqref_pack_gguf.argtypes = [i32, vp, vp, i64, i64, vp]
    L.lqref_unpack_gguf.argtypes = [i32, vp, i64, i64, vp, vp]
    L.lqref_quantize.argtypes = [i32, vp, i32, i64, i64, vp, vp]
    L.lqref_gemv.argtypes = [i32, vp, vp, vp, i32, i64, i64, vp, i64, vp, vp, i32]
    L.lqref_quantize_act.argtypes = [vp, i32, i64, i64, vp, vp, vp]
    L.lqref_gemv_q8act.argtypes = [i32, vp, vp, vp, vp, i64, i64, i64, vp, vp, i32]
    L.lqref_gemm.argtypes = [i32, vp, vp, vp, i32, i64, i64, i64,
                             vp, i64, vp, i64, i32, vp, vp, i32]
    return L


def _p(a):
    return None if a is None else a.ctypes.data


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what} rejected its arguments (rc={rc})")


def _xdt(x: np.ndarray):
    if x.dtype == np.float32:
        return F32, np.ascontiguousarray(x)
    if x.dtype == np.float16:
        return F16, np.ascontiguousarray(x).view(np.uint16)
    raise TypeError(f"x must be float32 or float16, got {x.dtype}")


class Oracle:
    """One loaded build of the oracle library."""

    def __init__(self, path: str):
        self.path = path
        self.L = _bind(ctypes.CDLL(path))

    def half_to_double(self, h: int) -> float:
        return self.L.lqref_half_to_double(int(h))

    def double_to_half(self, v: float) -> int:
        return int(self.L.lqref_double_to_half(float(v)))

    def block_elems(self, fmt) -> int:
        return self.L.lqref_block_elems(fmt)

    def gguf_block_bytes(self, fmt) -> int:
        return self.L.lqref_gguf_block_bytes(fmt)

    def dequant(self, fmt, w, scales, N, K):
        out = np.empty((N, K), np.float64)
        _check(self.L.lqref_dequant(fmt, _p(w), _p(scales), N, K, _p(out)), "dequant")
        return out

    def dequant_f32(self, fmt, w, scales, N, K):
        out = np.empty((N, K), np.float32)
        _check(self.L.lqref_dequant_f32(fmt, _p(w), _p(scales), N, K, _p(out)), "dequant_f32")
        return out

    def dequant_f16(self, fmt, w, scales, N, K):
        """Returns the fp16 bit patterns (uint16)."""
        out = np.empty((N, K), np.uint16)
        _check(self.L.lqref_dequant_f16(fmt, _p(w), _p(scales), N, K, _p(out)), "dequant_f16")
        return out

    def pack_gguf(self, fmt, codes, scales_bits, N, K):
        codes = np.ascontiguousarray(codes, dtype=np.int8)
        scales_bits = np.ascontiguousarray(scales_bits, dtype=np.uint16)
        out = np.empty(N * (K // 32) * self.gguf_block_bytes(fmt), np.uint8)
        _check(self.L.lqref_pack_gguf(fmt, _p(codes), _p(scales_bits), N, K, _p(out)), "pack_gguf")
        return out

    def quantize(self, fmt, src, N, K, sdt=None):
        """Load-time quantization of a row-major N x K matrix (see lqref.h).
        src: float32 or float16 array, or uint16 bf16 bit patterns with
        sdt=BF16.  Returns (GGUF bytes, None) for Q4_0 / Q8_0 and
        (int8 codes, fp32 scales) for I8B64 / I8B32, the forms the other
        calls take."""
        if sdt is None:
            sdt, src = _xdt(src)
        else:
            src = np.ascontiguousarray(src)
        if fmt in PLANAR:
            codes = np.empty(N * K, np.int8)
            scales = np.empty(N * (K // self.block_elems(fmt)), np.float32)
            _check(self.L.lqref_quantize(fmt, _p(src), sdt, N, K, _p(codes), _p(scales)), "quantize")
            return codes, scales
        out = np.empty(N * (K // 32) * self.gguf_block_bytes(fmt), np.uint8)
        _check(self.L.lqref_quantize(fmt, _p(src), sdt, N, K, _p(out), None), "quantize")
        return out, None

    def unpack_gguf(self, fmt, aos, N, K):
        codes = np.empty((N, K), np.int8)
        scales = np.empty((N, K // 32), np.uint16)
        _check(self.L.lqref_unpack_gguf(fmt, _p(aos), N, K, _p(codes), _p(scales)), "unpack_gguf")
        return codes, scales

    def quantize_act(self, X, M, K):
        """Per-matmul activation quantization of M x K activations (float32
        or float16): returns (q int8 M x K, s fp32 M x K/32, sum int32 M x K/32)."""
        xdt, xa = _xdt(np.asarray(X).reshape(-1))
        q = np.empty((M, K), np.int8)
        s = np.empty((M, K // 32), np.float32)
        t = np.empty((M, K // 32), np.int32)
        _check(self.L.lqref_quantize_act(_p(xa), xdt, M, K, _p(q), _p(s), _p(t)), "quantize_act")
        return q, s, t

    def gemv_q8act(self, fmt, w, scales, q, s, M, N, K, nthreads=None):
        """Integer-dot product on quantized activations: (Y, S) in float64, M x N."""
        q = np.ascontiguousarray(q, np.int8)
        s = np.ascontiguousarray(s, np.float32)
        Y = np.empty((M, N), np.float64)
        S = np.empty((M, N), np.float64)
        nt = nthreads or os.cpu_count() or 1
        _check(self.L.lqref_gemv_q8act(fmt, _p(w), _p(scales), _p(q), _p(s), M, N, K, _p(Y), _p(S), nt),
               "gemv_q8act")
        return Y, S

    def gemv(self, fmt, w, scales, x, N, K, rows=None, nthreads=None):
        """Returns (y, S) in float64 for the selected rows (all rows by default)."""
        xdt, xa = _xdt(x)
        if rows is None:
            nrows, rp = N, None
        else:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            nrows, rp = len(rows), rows
        y = np.empty(nrows, np.float64)
        S = np.empty(nrows, np.float64)
        nt = nthreads or os.cpu_count() or 1
        _check(self.L.lqref_gemv(fmt, _p(w), _p(scales), _p(xa), xdt, N, K, _p(rp), nrows,
                                 _p(y), _p(S), nt), "gemv")
        return y, S

    def gemm(self, fmt, w, scales, X, M, N, K, ms=None, ns=None, round_w_f16=False,
             nthreads=None):
        """Returns (Y, S) in float64, shape len(ms) x len(ns)  (Y = X W^T)."""
        xdt, xa = _xdt(X)
        ms = np.arange(M, dtype=np.int64) if ms is None else np.ascontiguousarray(ms, np.int64)
        ns = np.arange(N, dtype=np.int64) if ns is None else np.ascontiguousarray(ns, np.int64)
        Y = np.empty((len(ms), len(ns)), np.float64)
        S = np.empty((len(ms), len(ns)), np.float64)
        nt = nthreads or os.cpu_count() or 1
        _check(self.L.lqref_gemm(fmt, _p(w), _p(scales), _p(xa), xdt, M, N, K, _p(ms), len(ms),
                                 _p(ns), len(ns), int(bool(round_w_f16)), _p(Y), _p(S), nt),
               "gemm")
        return Y, S


_default = None


def default() -> Oracle:
    """The oracle built from lqref.cpp in this directory (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build()
        _default = Oracle(_LIB)
    return _default


def build_variant(src_text: str, out_dir: str) -> Oracle:
    """Compile a modified copy of the oracle source (used by the tests that
    plant a mistake in the oracle and check that the pins catch it)."""
    src = os.path.join(out_dir, "lqref_variant.cpp")
    hdr = os.path.join(out_dir, "lqref.h")
    with open(src, "w") as f:
        f.write(src_text)
    with open(os.path.join(_HERE, "lqref.h")) as f, open(hdr, "w") as g:
        g.write(f.read())
    so = os.path.join(out_dir, "liblqref_variant.so")
    subprocess.run(["g++", "-O1", "-std=c++17", "-fPIC", "-shared", "-pthread",
                    "-ffp-contract=off", "-o", so, src], check=True)
    return Oracle(so)


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()
