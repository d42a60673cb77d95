"""Grouped prefill GEMM (lq_gemm_batch): weight matrices that share X, M and K.

Each descriptor's Y must be what lq_gemm gives for that matrix alone (the
same bits, unless lq_gemm splits that matrix's K, which a grouped launch
never does) and within the GEMM bar of the exact product.  Every format runs
a group as one launch; Q4_0 and Q8_0 can pick the wider 192-row weight tile when the narrower one would need a second round of
workgroups (e.g. M = 512 over two 8200-row or two 11008-row matrices on a
256-CU part); the shapes below cover that path, ragged N (not a multiple of
64 or of 192), ragged M, and K of a few blocks (fewer steps than the copy
ring is deep).
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


def gemm_batch(fmt, Ws, X, M, Ns, K):
    Xd = to_device(X)
    Ys = [gu.guarded(M * N) for N in Ns]
    ws_bytes = max(lq.lq_gemm_workspace_bytes(gu.FMT[fmt], M, N, K) for N in Ns)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda") if ws_bytes else None
    lq.lq_gemm_batch(gu.FMT[fmt], Xd, M, K, list(zip(Ws, Ys, Ns)), ws=ws, ws_bytes=ws_bytes)
    torch.cuda.synchronize()
    out = []
    for Y, N in zip(Ys, Ns):
        gu.check_guard(Y, M * N)
        out.append(Y[:M * N].cpu().numpy().reshape(M, N))
    return out


def sample(M, N, rng, edges_m=(), edges_n=()):
    ms = np.unique(np.clip(np.concatenate([[0, M - 1], list(edges_m), rng.integers(0, M, 24)]), 0, M - 1))
    ns = np.unique(np.clip(np.concatenate([[0, N - 1], list(edges_n), rng.integers(0, N, 96)]), 0, N - 1))
    return ms, ns


GROUPS = [
    # (fmt, M, [N...], K)
    ("q4_0", 512, [8200, 8200], 256),         # wide tile: 2 rounds of 128-row tiles, 1 of 192-row
    ("q4_0", 300, [8200, 8264], 64),          # ragged M, two K blocks
    ("q4_0", 512, [64, 1000, 33, 4100], 96),  # four matrices, tiny and ragged N
    ("q4_0", 16, [128, 130], 2048),
    ("q8_0", 40, [70, 300], 512),
    ("q8_0", 512, [8200, 8264], 128),         # Q8_0 on the 192-row tile (five-slot copy ring)
    ("i8b64", 33, [256, 65], 1024),
    ("i8b64", 512, [8200, 8264], 128),        # two 64-element units per row
    ("i8b64", 300, [64, 1000, 33, 4100], 192),  # four matrices, an odd number of units
    ("i8b32", 512, [8200, 8264], 96),
    ("i8b32", 33, [256, 65], 1024),
]


@pytest.mark.parametrize("fmt,M,Ns,K", GROUPS)
def test_batch_parity_and_same_bits_as_single(oracle, fmt, M, Ns, K):
    say("gemm batch", fmt, M, Ns, K)
    mats = [make(fmt, 9100 + 7 * i + N, N, K) for i, N in enumerate(Ns)]
    Wd = [gu.upload(fmt, w, s, N, K) for (w, s), N in zip(mats, Ns)]
    X = lqgen.activations(9200 + K + M, M * K, np.float16).reshape(M, K)
    Ys = gemm_batch(fmt, Wd, X, M, Ns, K)
    rng = np.random.default_rng(M + K + len(Ns))
    for (w, s), W1, Y, N in zip(mats, Wd, Ys, Ns):
        # Same bits as lq_gemm alone unless that splits K (a grouped Q4_0 /
        # Q8_0 launch never does); within the bar either way.
        single = gu.gemm(W1, X, M, N, K, fmt)
        if len(Ns) == 1 or lq.lq_gemm_workspace_bytes(gu.FMT[fmt], M, N, K) == 0:
            assert np.array_equal(Y.view(np.uint32), single.view(np.uint32)), (fmt, M, N, K, "differs from lq_gemm")
        ms, ns = sample(M, N, rng, (255, 256), (63, 64, 127, 128, 191, 192))
        Yr, S = oracle.gemm(ORACLE_FMT[fmt], w, s, X, M, N, K, ms=ms, ns=ns)
        r = gu.ratio(Y[np.ix_(ms, ns)], Yr, S, gu.GEMM_REL, gu.GEMM_ABS)
        assert r <= 1.0, (fmt, M, N, K, r)


def test_batch_one_hot_rows_pin_tile():
    """X rows e_k: Y[m, :] is column k of the fp16 weight tile, bitwise, for
    every matrix of a group that takes the 192-row tile."""
    M, K = 512, 128
    Ns = [8200, 8200]
    mats = [make("q4_0", 9300 + i, N, K) for i, N in enumerate(Ns)]
    Wd = [gu.upload("q4_0", w, None, N, K) for (w, _), N in zip(mats, Ns)]
    ks = np.arange(M) % K
    X = np.zeros((M, K), np.float16)
    X[np.arange(M), ks] = 1.0
    Ys = gemm_batch("q4_0", Wd, X, M, Ns, K)
    for W1, Y, N in zip(Wd, Ys, Ns):
        t = torch.empty(N * K, dtype=torch.uint16, device="cuda")
        lq.lq_dequant_f16(lq.LQ_Q4_0, W1, t, N, K)
        torch.cuda.synchronize()
        tile = t.cpu().numpy().view(np.float16).reshape(N, K).astype(np.float32)
        assert np.array_equal(Y, tile[:, ks].T), N


@pytest.mark.slow
def test_fused_gate_up_matches_separate_launches(oracle):
    """The prefill FFN's gate and up projections (11008 x 2048, M = 512) in
    one launch: the same bits as two lq_gemm calls, and sampled outputs at
    the GEMM bar."""
    wl = lqgen.q4_0_prefill_ffn_2048x11008(512)
    M = wl.M
    gate, up = wl.mats[0], wl.mats[1]
    assert gate.xkey == up.xkey
    X = wl.x(gate.xkey)
    ws = [m.generate()[0] for m in (gate, up)]
    Wd = [gu.upload("q4_0", w, None, m.N, m.K) for w, m in zip(ws, (gate, up))]
    say("gemm fused gate+up", M, gate.N, gate.K)
    Ys = gemm_batch("q4_0", Wd, X, M, [gate.N, up.N], gate.K)
    rng = np.random.default_rng(7)
    for w, W1, Y, m in zip(ws, Wd, Ys, (gate, up)):
        single = gu.gemm(W1, X, M, m.N, m.K)
        assert np.array_equal(Y.view(np.uint32), single.view(np.uint32)), m.name
        ms, ns = sample(M, m.N, rng, (255, 256), (191, 192, 11007))
        Yr, S = oracle.gemm(0, w, None, X, M, m.N, m.K, ms=ms, ns=ns)
        assert gu.ratio(Y[np.ix_(ms, ns)], Yr, S, gu.GEMM_REL, gu.GEMM_ABS) <= 1.0, m.name
