"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no part of the product's arithmetic: it only draws random
numbers and lays them out as input buffers (GGUF array-of-blocks bytes for
Q4_0 / Q8_0, separate code and scale planes for int8 block-64, and fp32 or fp16
activations).  Both the HIP path and the oracle consume what it returns.

Random source: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), used counter-style: draw i of stream s is
mix64(s + (i + 1) * 0x9E3779B97F4A7C15).  Normals: Box-Muller (1958), cosine
branch, from two 53-bit uniforms.  Rounding of drawn values to fp16 / fp32 is
numpy's round-to-nearest-even cast.

Workload shapes (rows N x reduction K) follow the public configurations of the
models the pages run: SmolLM2-360M and SmolLM2-1.7B, Qwen2.5-0.5B and
Qwen2.5-3B ("lean" page, model table) and TinyLlama-1.1B ("wgpu-llm" page,
"Tested with"); value distributions are fixed synthetic recipes.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

Q4_0, Q8_0, I8B64, I8B32 = "q4_0", "q8_0", "i8b64", "i8b32"


def splitmix64(seed: int, n: int, start: int = 0) -> np.ndarray:
    """Draws start .. start+n-1 of the SplitMix64 stream seeded with `seed`."""
    with np.errstate(over="ignore"):
        i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform53(seed: int, n: int, start: int = 0) -> np.ndarray:
    """Uniform doubles k * 2^-53, k in [0, 2^53)."""
    return (splitmix64(seed, n, start) >> np.uint64(11)).astype(np.float64) * 2.0 ** -53


def normal(seed: int, n: int) -> np.ndarray:
    """n standard normals (float64), Box-Muller on draws (2i, 2i+1)."""
    u = uniform53(seed, 2 * n)
    u1 = u[0::2] + 2.0 ** -53          # (0, 1]: keeps log finite
    u2 = u[1::2]
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def random_bytes(seed: int, n: int, start_draw: int = 0) -> np.ndarray:
    nd = (n + 7) // 8
    return splitmix64(seed, nd, start_draw).view(np.uint8)[:n].copy()


def int8_sym127(seed: int, n: int) -> np.ndarray:
    """n int8 values uniform on -127..127 (bytes equal to 0x80 are rejected)."""
    out = np.empty(n, np.int8)
    got, draw = 0, 0
    while got < n:
        need = n - got
        nb = need + need // 128 + 64
        b = random_bytes(seed, nb, start_draw=draw)
        draw += (nb + 7) // 8
        b = b[b != 0x80].view(np.int8)[:need]
        out[got:got + len(b)] = b
        got += len(b)
    return out


def fp16_scales(seed: int, n: int, c: float) -> np.ndarray:
    """fp16 scale bits: RN_fp16(|z| * c), z ~ N(0,1)."""
    return (np.abs(normal(seed, n)) * c).astype(np.float16).view(np.uint16)


def fp32_scales(seed: int, n: int, c: float) -> np.ndarray:
    """fp32 scales: RN_fp32(|z| * c)."""
    return (np.abs(normal(seed, n)) * c).astype(np.float32)


def q4_0_aos(seed: int, N: int, K: int, c: float = 0.02) -> np.ndarray:
    """GGUF Q4_0 array-of-blocks bytes: per block fp16 d (LE) + 16 code bytes.
    Uniform random code bytes give two independent uniform 0..15 nibbles."""
    assert K % 32 == 0
    nblk = N * (K // 32)
    blk = np.empty((nblk, 18), np.uint8)
    blk[:, 0:2] = fp16_scales(seed * 2 + 1, nblk, c).view(np.uint8).reshape(nblk, 2)
    blk[:, 2:18] = random_bytes(seed * 2, nblk * 16).reshape(nblk, 16)
    return blk.reshape(-1)


def q8_0_aos(seed: int, N: int, K: int, c: float = 0.005) -> np.ndarray:
    """GGUF Q8_0 array-of-blocks bytes: per block fp16 d (LE) + 32 int8 codes."""
    assert K % 32 == 0
    nblk = N * (K // 32)
    blk = np.empty((nblk, 34), np.uint8)
    blk[:, 0:2] = fp16_scales(seed * 2 + 1, nblk, c).view(np.uint8).reshape(nblk, 2)
    blk[:, 2:34] = int8_sym127(seed * 2, nblk * 32).view(np.uint8).reshape(nblk, 32)
    return blk.reshape(-1)


def i8b64_planes(seed: int, N: int, K: int, c: float = 0.003):
    """int8 block-64 planes: codes (N*K int8, -127..127), scales (N*K/64 fp32)."""
    return i8_planes(seed, N, K, 64, c)


def i8_planes(seed: int, N: int, K: int, block: int, c: float = 0.003):
    """int8 planes with fp32 scales per `block` codes of a row: codes (N*K
    int8, -127..127), scales (N*K/block fp32)."""
    assert K % block == 0
    codes = int8_sym127(seed * 2, N * K)
    scales = fp32_scales(seed * 2 + 1, N * (K // block), c)
    return codes, scales


def activations(seed: int, n: int, dtype) -> np.ndarray:
    return normal(seed, n).astype(dtype)


def digest(a: np.ndarray) -> str:
    return hashlib.blake2b(np.ascontiguousarray(a).view(np.uint8).tobytes(), digest_size=8).hexdigest()


# ---------------------------------------------------------------------------
# Workload recipes
# ---------------------------------------------------------------------------

def seed_of(cfg: int, layer: int, mat: int) -> int:
    return 0x1A000000 + ((cfg * 64 + layer) * 16 + mat) * 16


@dataclass
class Mat:
    """One quantized matrix of a workload (generated on demand)."""
    name: str
    fmt: str
    N: int
    K: int
    seed: int
    scale_c: float
    xkey: str                 # which activation vector multiplies it

    def generate(self):
        """Returns (w, scales): GGUF bytes and None, or codes and fp32 scales."""
        if self.fmt == Q4_0:
            return q4_0_aos(self.seed, self.N, self.K, self.scale_c), None
        if self.fmt == Q8_0:
            return q8_0_aos(self.seed, self.N, self.K, self.scale_c), None
        return i8_planes(self.seed, self.N, self.K, 64 if self.fmt == I8B64 else 32, self.scale_c)

    @property
    def packed_bytes(self) -> int:
        """Bytes of weight data (codes + scales); identical for GGUF and planes."""
        per = {Q4_0: 18 / 32, Q8_0: 34 / 32, I8B64: 68 / 64, I8B32: 36 / 32}[self.fmt]
        return int(self.N * self.K * per)


@dataclass
class Workload:
    name: str
    mats: list
    xs: dict = field(default_factory=dict)   # key -> (seed, length, numpy dtype)
    M: int = 1                                # tokens (1 = decode GEMV)

    def x(self, key):
        seed, n, dt = self.xs[key]
        return activations(seed, n * self.M, dt).reshape(self.M, n) if self.M > 1 \
            else activations(seed, n, dt)

    @property
    def weight_bytes(self) -> int:
        return sum(m.packed_bytes for m in self.mats)


def q4_0_ffn_2560x960() -> Workload:
    """Q4_0 GEMV, 2560 x 960 (SmolLM2-360M FFN), codes U{0..15},
    d = RN16(|z| 0.02), x fp32 N(0,1), batch 1."""
    s = seed_of(0, 0, 0)
    return Workload("q4_0_gemv_2560x960",
                    [Mat("ffn", Q4_0, 2560, 960, s, 0.02, "x")],
                    {"x": (s + 15, 960, np.float32)})


def q8_0_layer_2048(layer: int = 0) -> Workload:
    """Q8_0 GEMV set of one decoder layer, hidden 2048 / FFN 8192
    (SmolLM2-1.7B): q,k,v,o 2048x2048; gate,up 8192x2048; down 2048x8192.
    Codes U{-127..127}, d = RN16(|z| 0.005), x fp32 N(0,1).  One x shared by
    q,k,v; one for o; one shared by gate,up; one for down."""
    mats = []
    shapes = [("q", 2048, 2048, "x_attn"), ("k", 2048, 2048, "x_attn"),
              ("v", 2048, 2048, "x_attn"), ("o", 2048, 2048, "x_o"),
              ("gate", 8192, 2048, "x_ffn"), ("up", 8192, 2048, "x_ffn"),
              ("down", 2048, 8192, "x_down")]
    for i, (nm, N, K, xk) in enumerate(shapes):
        mats.append(Mat(nm, Q8_0, N, K, seed_of(1, layer, i), 0.005, xk))
    base = seed_of(1, layer, 15)
    xs = {"x_attn": (base + 1, 2048, np.float32), "x_o": (base + 2, 2048, np.float32),
          "x_ffn": (base + 3, 2048, np.float32), "x_down": (base + 4, 8192, np.float32)}
    return Workload(f"q8_0_layer_h2048_f8192_l{layer}", mats, xs)


def q4_0_lmhead_151936x896(with_ffn: bool = True) -> Workload:
    """Q4_0 GEMV LM head 151936 x 896 (Qwen2.5-0.5B) plus its 4864 x 896
    gate and up matrices; distributions as the 2560 x 960 case."""
    mats = [Mat("lm_head", Q4_0, 151936, 896, seed_of(2, 0, 0), 0.02, "x")]
    if with_ffn:
        mats += [Mat("gate", Q4_0, 4864, 896, seed_of(2, 0, 1), 0.02, "x"),
                 Mat("up", Q4_0, 4864, 896, seed_of(2, 0, 2), 0.02, "x")]
    return Workload("q4_0_lmhead_151936x896", mats, {"x": (seed_of(2, 0, 15) + 1, 896, np.float32)})


def i8b64_tinyllama_layer(layer: int) -> Workload:
    """int8 block-64 GEMV set of one TinyLlama-1.1B layer: hidden 2048,
    FFN 5632, 32 q / 4 kv heads of 64 (k, v are 256 x 2048); fp32 block scales
    RN32(|z| 0.003); x fp16 N(0,1)."""
    shapes = [("q", 2048, 2048, "x_attn"), ("k", 256, 2048, "x_attn"),
              ("v", 256, 2048, "x_attn"), ("o", 2048, 2048, "x_o"),
              ("gate", 5632, 2048, "x_ffn"), ("up", 5632, 2048, "x_ffn"),
              ("down", 2048, 5632, "x_down")]
    mats = [Mat(nm, I8B64, N, K, seed_of(3, layer, i), 0.003, xk)
            for i, (nm, N, K, xk) in enumerate(shapes)]
    base = seed_of(3, layer, 15)
    xs = {"x_attn": (base + 1, 2048, np.float16), "x_o": (base + 2, 2048, np.float16),
          "x_ffn": (base + 3, 2048, np.float16), "x_down": (base + 4, 5632, np.float16)}
    return Workload(f"i8b64_tinyllama_l{layer}", mats, xs)


TINYLLAMA_LAYERS = 22


def q4_0_prefill_ffn_2048x11008(M: int = 512) -> Workload:
    """Q4_0 prefill GEMM over an FFN of hidden 2048 / intermediate 11008
    (Qwen2.5-3B): gate, up 11008 x 2048 and down 2048 x 11008; X fp16 N(0,1),
    M tokens; weight distributions as the 2560 x 960 case."""
    mats = [Mat("gate", Q4_0, 11008, 2048, seed_of(4, 0, 0), 0.02, "x_ffn"),
            Mat("up", Q4_0, 11008, 2048, seed_of(4, 0, 1), 0.02, "x_ffn"),
            Mat("down", Q4_0, 2048, 11008, seed_of(4, 0, 2), 0.02, "x_down")]
    base = seed_of(4, 0, 15)
    xs = {"x_ffn": (base + 1, 2048, np.float16), "x_down": (base + 2, 11008, np.float16)}
    return Workload(f"q4_0_prefill_ffn_m{M}", mats, xs, M=M)


def multi_token(wl: Workload, M: int) -> Workload:
    """The same matrices decoded for M tokens at once (a verification pass
    over M drafted tokens): every activation vector becomes an M x K fp16
    N(0,1) matrix drawn from the same seed."""
    xs = {k: (seed, n, np.float16) for k, (seed, n, _) in wl.xs.items()}
    return Workload(f"{wl.name}_m{M}", list(wl.mats), xs, M=M)
