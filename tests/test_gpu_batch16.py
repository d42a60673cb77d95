"""Grouped calls with more matrices than one launch takes: 18 descriptors per
call, run as a launch of 16 and one of 2 (needs an MI355X).

A grouped launch finds a workgroup's matrix by counting the entries of a
16-entry table of first workgroups that are not after it; these cases fill
every entry.  They cover the one-token GEMV with K unsplit, K split inside
16-wave workgroups and across them, the sub-tile kernel (few tiles of the
multi-part formats) and the multi-token GEMV, every output against the
oracle at the GEMV bar (|y - y_ref| <= 1e-4 * sum|w x| + 1e-6 per row).
"""
import sys

import numpy as np
import pytest
import torch

import gemm_q4_q8_int8_amd as lq
import lqgen
from gemm_q4_q8_int8_amd.device import to_device
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

ORACLE_FMT = {"q4_0": 0, "q8_0": 1, "i8b64": 2, "i8b32": 3}
COUNT = 18


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    lq.load()
    lq.lq_init()
    yield


def make(fmt, seed, N, K):
    if fmt == "q4_0":
        return lqgen.q4_0_aos(seed, N, K, 0.02), None
    if fmt == "q8_0":
        return lqgen.q8_0_aos(seed, N, K, 0.005), None
    return lqgen.i8_planes(seed, N, K, 64 if fmt == "i8b64" else 32, 0.003)


def shapes(kind):
    """18 (N, K) pairs.  small: a few ragged tiles each (the sub-tile kernel
    for the multi-part formats); split: K = 2048 and 8192 alternating, enough
    tiles that K splits inside 16-wave workgroups and, for K = 8192, across
    them."""
    if kind == "small":
        return [(64 + 37 * i, 512) for i in range(COUNT)]
    return [(512 + 64 * (i % 5) + 7 * i, 2048 if i % 2 == 0 else 8192) for i in range(COUNT)]


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0", "i8b64", "i8b32"])
@pytest.mark.parametrize("kind", ["small", "split"])
def test_gemv_batch_18(oracle, fmt, kind):
    say("gemv batch 18", fmt, kind)
    mats, descs, outs, keep = [], [], [], []
    for i, (N, K) in enumerate(shapes(kind)):
        w, s = make(fmt, 100 + i, N, K)
        x = lqgen.activations(200 + i, K, np.float32)
        Wd, xd, y = gu.upload(fmt, w, s, N, K), to_device(x), gu.guarded(N)
        mats.append((w, s, x, N, K))
        descs.append((gu.FMT[fmt], Wd, xd, y, N, K))
        outs.append(y)
        keep.append((Wd, xd))
    lq.lq_gemv_batch(descs, ws=gu.gemv_ws())
    torch.cuda.synchronize()
    for i, ((w, s, x, N, K), y) in enumerate(zip(mats, outs)):
        gu.check_guard(y, N)
        yr, S = oracle.gemv(ORACLE_FMT[fmt], w, s, x, N, K)
        r = gu.ratio(y[:N].cpu().numpy(), yr, S, gu.GEMV_REL, gu.GEMV_ABS)
        assert r <= 1.0, (fmt, kind, i, N, K, r)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("M", [3, 8])
def test_gemv_multi_batch_18(oracle, fmt, M):
    """18 multi-token descriptors in one call (few-token GEMV at M = 3, the
    multi-token matrix-core kernel at M = 8), every output."""
    say("gemv multi batch 18", fmt, M)
    mats, descs, outs, keep = [], [], [], []
    for i, (N, K) in enumerate(shapes("split")):
        K = 2048 if K > 2048 else K
        w, s = make(fmt, 300 + i, N, K)
        X = lqgen.activations(400 + i, M * K, np.float16).reshape(M, K)
        Wd, Xd, Y = gu.upload(fmt, w, s, N, K), to_device(X), gu.guarded(M * N)
        mats.append((w, s, X, N, K))
        descs.append((gu.FMT[fmt], Wd, Xd, Y, M, N, K))
        outs.append(Y)
        keep.append((Wd, Xd))
    lq.lq_gemv_multi_batch(descs, ws=gu.gemv_ws())
    torch.cuda.synchronize()
    for i, ((w, s, X, N, K), Y) in enumerate(zip(mats, outs)):
        gu.check_guard(Y, M * N)
        Yr, S = oracle.gemm(ORACLE_FMT[fmt], w, s, X, M, N, K)
        r = gu.ratio(Y[:M * N].cpu().numpy().reshape(M, N), Yr, S, gu.GEMV_REL, gu.GEMV_ABS)
        assert r <= 1.0, (fmt, M, i, N, K, r)
