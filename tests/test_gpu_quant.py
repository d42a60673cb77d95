"""GPU parity of lq_quantize (load-time block quantization) with the oracle.

Codes and scales are integer / bit-pattern results of the same IEEE fp32
steps on both sides, so the packed bytes must be identical.  The oracle's
output (GGUF blocks or code / scale planes) is packed with the library's own
repack / pack calls, whose byte-exactness the layout tests pin.
"""
import sys

import numpy as np
import pytest
import torch

import gemm_q4_q8_int8_amd as lq
import lqgen
from gemm_q4_q8_int8_amd.device import empty_packed, to_device
from tests import gpu_util as gu
from tests.test_gpu_parity import ORACLE_FMT

pytestmark = pytest.mark.gpu

SDT = {"f32": lq.LQ_F32, "f16": lq.LQ_F16, "bf16": lq.LQ_BF16}


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    lq.load()
    lq.lq_init()
    yield


def source(seed, N, K, sdt):
    """N x K weights with special blocks in the first rows: ties after
    division, zero blocks, equal magnitudes of both signs, tiny values
    (fp16 scale near or below its normal range), one dominant element."""
    w = (lqgen.activations(seed, N * K, np.float32) * 0.05).reshape(N, K)
    if N >= 6 and K >= 64:
        w[0, :32] = np.arange(32, dtype=np.float32) * 0.5 - 7.75        # many halves
        w[0, 32:64] = 0.0
        w[1, :32] = np.where(np.arange(32) % 2 == 0, 3.0, -3.0)           # +-max ties
        w[2, :32] = np.linspace(-1e-6, 1e-6, 32, dtype=np.float32)       # subnormal fp16 scale
        w[3, :32] = 1e-9
        w[4, :64] = 0.01
        w[4, 5] = 40.0                                                    # one dominant element
        w[5, :32] = np.float32(127.0) * np.arange(-16, 16, dtype=np.float32) / 16
    if sdt == "f32":
        return w, w
    if sdt == "f16":
        h = w.astype(np.float16)
        return h, h
    bits = (w.view(np.uint32) >> 16).astype(np.uint16)                    # exact bf16 values
    return bits, bits


SHAPES = [(1, 32), (6, 64), (65, 96), (130, 256), (7, 2048), (64, 896)]


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0", "i8b64", "i8b32"])
@pytest.mark.parametrize("sdt", ["f32", "f16", "bf16"])
def test_quantize_bitwise(oracle, fmt, sdt):
    for N, K in SHAPES:
        if fmt == "i8b64" and K % 64:
            continue
        say("quantize", fmt, sdt, N, K)
        host, ref_src = source(300 + N + K, N, K, sdt)
        src = to_device(host)
        Wd = empty_packed(gu.FMT[fmt], N, K)
        Wd.fill_(0xAB)
        lq.lq_quantize(gu.FMT[fmt], src, Wd, N, K, sdt=SDT[sdt])
        torch.cuda.synchronize()
        q, s = oracle.quantize(ORACLE_FMT[fmt], ref_src, N, K, sdt=2 if sdt == "bf16" else None)
        want = gu.upload(fmt, q, s, N, K)
        cb = N * K // 2 if fmt == "q4_0" else N * K
        off = lq.lq_scale_offset(gu.FMT[fmt], N, K)
        got, exp = Wd.cpu().numpy(), want.cpu().numpy()
        assert np.array_equal(got[:cb], exp[:cb]), (fmt, sdt, N, K, "codes")
        assert np.array_equal(got[off:], exp[off:]), (fmt, sdt, N, K, "scales")


def test_quantize_then_gemv(oracle):
    """fp32 weights quantized on the GPU and multiplied there agree with the
    oracle's GEMV over the oracle's quantization of the same weights."""
    N, K = 300, 2048
    for fmt in ("q4_0", "q8_0", "i8b64", "i8b32"):
        say("quantize + gemv", fmt, N, K)
        w = (lqgen.activations(77, N * K, np.float32) * 0.02).reshape(N, K)
        Wd = empty_packed(gu.FMT[fmt], N, K)
        lq.lq_quantize(gu.FMT[fmt], to_device(w), Wd, N, K)
        x = lqgen.activations(78, K, np.float32)
        y = gu.gemv(fmt, Wd, x, N, K)
        q, s = oracle.quantize(ORACLE_FMT[fmt], w, N, K)
        yr, S = oracle.gemv(ORACLE_FMT[fmt], q, s, x, N, K)
        assert gu.ratio(y, yr, S, gu.GEMV_REL, gu.GEMV_ABS) <= 1.0, fmt


@pytest.fixture(scope="module")
def x_max_k():
    return lqgen.activations(4096, 1 << 25, np.float32)


@pytest.mark.slow
@pytest.mark.parametrize("fmt", ["q4_0", "q8_0", "i8b64", "i8b32"])
def test_max_k_full_tile(oracle, fmt, x_max_k):
    """K at the documented maximum (2^25) with a full 64-row tile: the 32-bit
    offsets inside a tile reach their largest values.  Weights are generated
    and quantized on the GPU; the oracle quantizes the same fp16 rows on the
    host (the quantizers agree bit for bit) and checks sampled rows of the
    GEMV (K split across many workgroups) and of a two-token multi-token
    GEMV."""
    N, K = 64, 1 << 25
    say("max K", fmt, N, K)
    g = torch.Generator(device="cuda")
    g.manual_seed(2024)
    W16 = torch.randn(N, K, dtype=torch.float16, device="cuda", generator=g) * 0.05
    Wd = empty_packed(gu.FMT[fmt], N, K)
    lq.lq_quantize(gu.FMT[fmt], W16, Wd, N, K)
    x = x_max_k
    y = gu.gemv(fmt, Wd, x, N, K)
    # two tokens through the multi-token GEMV on the same weights
    x16 = x.astype(np.float16)
    X2 = np.stack([x16, -x16[::-1]])
    Y2 = gu.gemv_multi(fmt, Wd, X2, 2, N, K)
    for row in (0, 37, 63):
        w_row = W16[row].cpu().numpy()
        q, s = oracle.quantize(ORACLE_FMT[fmt], w_row, 1, K)
        yr, S = oracle.gemv(ORACLE_FMT[fmt], q, s, x, 1, K)
        r = gu.ratio(y[row:row + 1], yr, S, gu.GEMV_REL, gu.GEMV_ABS)
        assert r <= 1.0, (fmt, row, r)
        Yr, S2 = oracle.gemm(ORACLE_FMT[fmt], q, s, X2, 2, 1, K)
        r2 = gu.ratio(Y2[:, row:row + 1], Yr, S2, gu.GEMV_REL, gu.GEMV_ABS)
        assert r2 <= 1.0, (fmt, row, "multi", r2)
    del W16, Wd
    torch.cuda.empty_cache()
