"""Sub-tile GEMV: launches of Q8_0 or int8 block-64 matrices with rows of at
most 128 units and few 64-row tiles (at most one workgroup per CU once each
tile is split by rows) split each tile by rows across 2 (Q8_0) or 4 (int8
block-64) workgroups, each lane taking one 16-byte code part of a row.  The
shapes below all take that path on a 256-CU device.

Checked against the oracle at the GEMV bar (|y - y_ref| <= 1e-4 sum|w x| +
1e-6), on the int8 block-64 decoder layer's launches as a decoder runs them
(q/k/v grouped, o, gate/up grouped, down), on ragged tiles whose last
workgroups hold no rows, and with one-hot activations, which must give the
weight column exactly as lq_dequant_f32 unpacks it (one nonzero product per
row, every other term an exact zero: a wrong part, row or activation offset
shows up as a wrong or missing value).
"""
import numpy as np
import pytest
import torch

import gemm_q4_q8_int8_amd as lq
import lqgen
from gemm_q4_q8_int8_amd.device import to_device
from tests import gpu_util as gu
from tests.test_gpu_parity import ORACLE_FMT, make, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    lq.load()
    lq.lq_init()
    yield


# (fmt, N, K): ragged tiles (N % 64 leaves 1..63 rows, so some row groups of
# the last tile are empty), one-row matrices, one-unit rows, and the longest
# rows this path takes (128 units).
SUB_SHAPES = [
    ("q8_0", 1, 32), ("q8_0", 31, 64), ("q8_0", 33, 4096), ("q8_0", 65, 1024), ("q8_0", 96, 2048),
    ("q8_0", 4000, 512),
    ("i8b64", 1, 64), ("i8b64", 15, 64), ("i8b64", 17, 8192), ("i8b64", 70, 640), ("i8b64", 130, 2048),
    ("i8b64", 4050, 1024),
    ("i8b32", 1, 32), ("i8b32", 33, 4096), ("i8b32", 70, 640), ("i8b32", 4000, 512),
]


@pytest.mark.parametrize("fmt,N,K", SUB_SHAPES)
@pytest.mark.parametrize("xdt", [np.float32, np.float16], ids=["xf32", "xf16"])
def test_sub_tile_parity(oracle, fmt, N, K, xdt):
    say("gemv sub-tile", fmt, N, K, np.dtype(xdt).name)
    w, s = make(fmt, 5100 + N + K, N, K)
    x = lqgen.activations(5200 + K, K, xdt)
    Wd = gu.upload(fmt, w, s, N, K)
    y = gu.gemv(fmt, Wd, x, N, K)
    y2 = gu.gemv(fmt, Wd, x, N, K)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "not deterministic"
    yr, S = oracle.gemv(ORACLE_FMT[fmt], w, s, x, N, K)
    assert gu.ratio(y, yr, S, gu.GEMV_REL, gu.GEMV_ABS) <= 1.0


@pytest.mark.parametrize("fmt,N,K", [("q8_0", 70, 1024), ("i8b64", 70, 1024), ("i8b64", 129, 256),
                                      ("i8b32", 70, 1024)])
def test_sub_tile_one_hot_columns(fmt, N, K):
    say("gemv sub-tile one-hot", fmt, N, K)
    w, s = make(fmt, 5300 + N, N, K)
    Wd = gu.upload(fmt, w, s, N, K)
    out = torch.empty(N * K, dtype=torch.float32, device="cuda")
    lq.lq_dequant_f32(gu.FMT[fmt], Wd, out, N, K)
    torch.cuda.synchronize()
    full = out.cpu().numpy().reshape(N, K)
    for k in (0, 1, 15, 16, 17, 31, 32, 47, 48, 63, 64, K // 2 + 5, K - 1):
        for xdt in (np.float32, np.float16):
            x = np.zeros(K, xdt)
            x[k] = 1
            y = gu.gemv(fmt, Wd, x, N, K)
            assert np.array_equal(y.view(np.uint32), full[:, k].view(np.uint32)), (k, np.dtype(xdt).name)


def test_int8_decoder_layer_launches(oracle):
    """The int8 block-64 layer (h2048 / f5632, kv 256) launched as a decoder
    does: q/k/v in one call, o, gate/up in one call, down."""
    wl = lqgen.i8b64_tinyllama_layer(0)
    mats = {m.name: m for m in wl.mats}
    data = {n: m.generate() for n, m in mats.items()}
    Wd = {n: gu.upload("i8b64", c, sc, mats[n].N, mats[n].K) for n, (c, sc) in data.items()}
    xs = {k: wl.x(k) for k in wl.xs}
    xd = {k: to_device(v) for k, v in xs.items()}
    for group in (["q", "k", "v"], ["o"], ["gate", "up"], ["down"]):
        say("int8 layer launch", group)
        ys = {n: gu.guarded(mats[n].N) for n in group}
        lq.lq_gemv_batch([(lq.LQ_I8B64, Wd[n], xd[mats[n].xkey], ys[n], mats[n].N, mats[n].K) for n in group],
                         ws=gu.gemv_ws())
        torch.cuda.synchronize()
        for n in group:
            m = mats[n]
            gu.check_guard(ys[n], m.N)
            c, sc = data[n]
            yr, S = oracle.gemv(ORACLE_FMT["i8b64"], c, sc, xs[m.xkey], m.N, m.K)
            assert gu.ratio(ys[n][:m.N].cpu().numpy(), yr, S, gu.GEMV_REL, gu.GEMV_ABS) <= 1.0, n
