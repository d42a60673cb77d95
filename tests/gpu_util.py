"""Shared helpers of the GPU parity tests: upload, run through the C ABI,
compare with the oracle under the stated tolerances."""
import numpy as np
import torch

import gemm_q4_q8_int8_amd as lq
from gemm_q4_q8_int8_amd.device import to_device, upload_gguf, upload_planes

FMT = {"q4_0": lq.LQ_Q4_0, "q8_0": lq.LQ_Q8_0, "i8b64": lq.LQ_I8B64, "i8b32": lq.LQ_I8B32}
PLANAR = ("i8b64", "i8b32")   # int8 codes + fp32 scale planes
GUARD = 1024            # canary floats after every output buffer
SENTINEL = -12345.5

GEMV_REL, GEMV_ABS = 1e-4, 1e-6     # |y - y_ref| <= 1e-4 * sum|w x| + 1e-6 per row
GEMM_REL, GEMM_ABS = 2e-3, 1e-5     # |Y - Y_ref| <= 2e-3 * sum|w x| + 1e-5 per element


def upload(fmt: str, w, scales, N, K):
    if fmt in PLANAR:
        return upload_planes(FMT[fmt], w, scales, N, K)
    return upload_gguf(FMT[fmt], w, N, K)


def tiled_reference(fmt: str, codes_rows: np.ndarray, scales_rows: np.ndarray, N, K) -> np.ndarray:
    """Host construction of the packed layout that lq.h documents, from
    row-major planes: codes_rows (N, units, unit bytes) uint8, scales_rows
    (N, units) fp16 bits or fp32.  Rows go in tiles of 64 (the last may be
    shorter); inside a tile, unit by unit, 16-byte part by part, the rows'
    parts side by side; scales the same way, one per unit and row."""
    E = 64 if fmt == "i8b64" else 32
    P = {"q4_0": 1, "q8_0": 2, "i8b64": 4, "i8b32": 2}[fmt]
    nu = K // E
    out = np.zeros(lq.lq_packed_bytes(FMT[fmt], N, K), np.uint8)
    soff = lq.lq_scale_offset(FMT[fmt], N, K)
    codes_rows = np.ascontiguousarray(codes_rows).view(np.uint8).reshape(N, nu, P, 16)
    sc = np.ascontiguousarray(scales_rows).reshape(N, nu)
    sbytes = sc.dtype.itemsize
    cpos, spos = 0, soff
    for t0 in range(0, N, 64):
        nr = min(64, N - t0)
        blk = np.ascontiguousarray(codes_rows[t0:t0 + nr].transpose(1, 2, 0, 3)).reshape(-1)
        out[cpos:cpos + blk.size] = blk
        cpos += blk.size
        sb = np.ascontiguousarray(sc[t0:t0 + nr].T).view(np.uint8).reshape(-1)
        out[spos:spos + sb.size] = sb
        spos += sb.size
    assert cpos == (N * K // 2 if fmt == "q4_0" else N * K) and spos == out.size
    return out


def guarded(n, dtype=torch.float32):
    buf = torch.full((n + GUARD,), SENTINEL, dtype=dtype, device="cuda")
    return buf


def check_guard(buf, n):
    tail = buf[n:].cpu().numpy()
    assert np.all(tail == SENTINEL), "write past the end of the output buffer"


_WS = {}


def gemv_ws(key=0):
    """A GEMV split-K workspace (lq_gemv_workspace_bytes() bytes), one per key
    and device, filled with garbage once: the library needs no clearing."""
    dev = torch.cuda.current_device()
    if (dev, key) not in _WS:
        _WS[(dev, key)] = torch.full((lq.lq_gemv_workspace_bytes(),), 0xA5, dtype=torch.uint8, device="cuda")
    return _WS[(dev, key)]


def gemv(fmt: str, Wd, x: np.ndarray, N, K, ws=True):
    """y = W x through lq_gemv; ws=True passes the shared workspace (K may be
    split across workgroups), ws=None runs without one."""
    xd = to_device(x)
    y = guarded(N)
    lq.lq_gemv(FMT[fmt], Wd, xd, y, N, K, ws=gemv_ws() if ws is True else ws)
    torch.cuda.synchronize()
    check_guard(y, N)
    return y[:N].cpu().numpy()


def gemm(Wd, X: np.ndarray, M, N, K, fmt: str = "q4_0"):
    Xd = to_device(X)
    Y = guarded(M * N)
    ws_bytes = lq.lq_gemm_workspace_bytes(FMT[fmt], M, N, K)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda") if ws_bytes else None
    lq.lq_gemm(FMT[fmt], Wd, Xd, Y, M, N, K, ws=ws, ws_bytes=ws_bytes)
    torch.cuda.synchronize()
    check_guard(Y, M * N)
    return Y[:M * N].cpu().numpy().reshape(M, N)


def ratio(y, yref, S, rel, abs_):
    """max over elements of |y - y_ref| / (rel * S + abs_); parity holds when <= 1."""
    y = np.asarray(y, np.float64)
    assert np.all(np.isfinite(y)), "non-finite output"
    return float(np.max(np.abs(y - yref) / (rel * S + abs_))) if y.size else 0.0


def gemv_multi(fmt: str, Wd, X: np.ndarray, M, N, K, ws=True):
    Xd = to_device(X)
    Y = guarded(M * N)
    lq.lq_gemv_multi(FMT[fmt], Wd, Xd, Y, M, N, K, ws=gemv_ws() if ws is True else ws)
    torch.cuda.synchronize()
    check_guard(Y, M * N)
    return Y[:M * N].cpu().numpy().reshape(M, N)
