"""Device-memory plumbing around liblq (torch allocates, liblq converts).

upload_gguf:   host GGUF Q4_0 / Q8_0 array-of-blocks bytes -> device -> packed
               layout through lq_repack_gguf.
upload_planes: host code and scale planes -> device -> packed layout through
               lq_pack_planes (int8 block-64, or split Q4_0 / Q8_0 planes).
Buffers are 256-byte aligned torch allocations on the current device.
"""
from __future__ import annotations

import numpy as np
import torch

from . import lq_gguf_bytes, lq_pack_planes, lq_packed_bytes, lq_repack_gguf, _fmt


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def empty_packed(fmt, N, K, device="cuda") -> torch.Tensor:
    nbytes = lq_packed_bytes(_fmt(fmt), N, K)
    if nbytes == 0:
        raise ValueError(f"invalid packed shape fmt={fmt} N={N} K={K}")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def upload_gguf(fmt, aos: np.ndarray, N, K, device="cuda", stream=None) -> torch.Tensor:
    f = _fmt(fmt)
    if aos.nbytes != lq_gguf_bytes(f, N, K):
        raise ValueError(f"GGUF buffer has {aos.nbytes} bytes, expected {lq_gguf_bytes(f, N, K)}")
    src = to_device(aos.view(np.uint8), device)
    dst = empty_packed(f, N, K, device)
    lq_repack_gguf(f, src, dst, N, K, stream=stream)
    torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()
    del src
    return dst


def upload_planes(fmt, codes: np.ndarray, scales: np.ndarray, N, K, device="cuda",
                  stream=None) -> torch.Tensor:
    f = _fmt(fmt)
    c = to_device(codes.view(np.uint8), device)
    s = to_device(scales, device)
    dst = empty_packed(f, N, K, device)
    lq_pack_planes(f, c, s, dst, N, K, stream=stream)
    torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()
    del c, s
    return dst
