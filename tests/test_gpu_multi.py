"""GPU parity of the multi-token GEMV (lq_gemv_multi) against the CPU oracle.

Y[m, n] = sum_k w[n,k] X[m,k] for up to 16 tokens with fp16 activations.  The
bar is the single-token GEMV's, per output: |Y - Y_ref| <= 1e-4 * sum|w x| +
1e-6, since the weights are decoded exactly and only the fp32 sums round.
Shapes span several 64-row tiles, partial last tiles, one-block rows, K split
across workgroups, and every token count from 1 to 16.  Up to two tokens
(Q4_0) or four (Q8_0, int8 block-64) run on the single-token GEMV kernel
(each token row then equals lq_gemv of that row bit for bit); more on the
matrix-core kernel.
"""
import sys

import numpy as np
import pytest
import torch

import gemm_q4_q8_int8_amd as lq
import lqgen
from gemm_q4_q8_int8_amd.device import to_device
from tests import gpu_util as gu
from tests.test_gpu_parity import ORACLE_FMT, make, set_scales

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    lq.load()
    lq.lq_init()
    yield


# (fmt, M, N, K): tails in rows (N % 64) and tokens, single-block rows, long
# K (split across workgroups when N is small), and big-N single-slice cases.
# Q4_0 waves with 5 to 7 units load them as one batch of 7: K = 896 fills it,
# K = 704 (22 units: waves of 5 and 6) and 640 leave slots of it unused.
MULTI_SHAPES = [
    ("q4_0", 1, 1, 32), ("q4_0", 2, 5, 64), ("q4_0", 3, 67, 96), ("q4_0", 16, 64, 896),
    ("q4_0", 5, 130, 960), ("q4_0", 8, 300, 2048), ("q4_0", 13, 33, 11008), ("q4_0", 16, 2500, 896),
    ("q4_0", 4, 17, 25600), ("q4_0", 3, 129, 704), ("q4_0", 9, 3000, 640),
    ("q8_0", 1, 3, 32), ("q8_0", 2, 70, 512), ("q8_0", 7, 130, 2048), ("q8_0", 16, 64, 8192),
    ("q8_0", 11, 200, 5632), ("q8_0", 16, 1100, 1024),
    ("i8b64", 1, 1, 64), ("i8b64", 3, 77, 128), ("i8b64", 16, 256, 2048), ("i8b64", 6, 45, 5632),
    ("i8b64", 16, 130, 8192), ("i8b64", 9, 5, 30720), ("i8b64", 14, 1500, 512),
    # GEMV-kernel token counts: K split across workgroups, 16-wave workgroups, ragged tiles
    ("q4_0", 2, 17, 25600), ("q4_0", 2, 2500, 896), ("q4_0", 1, 200, 4096),
    ("q8_0", 2, 130, 8192), ("q8_0", 1, 200, 5632), ("q8_0", 3, 3000, 2048), ("q8_0", 4, 77, 4096),
    ("q8_0", 4, 8200, 1024),
    ("i8b64", 2, 45, 5632), ("i8b64", 1, 130, 8192), ("i8b64", 3, 1500, 512), ("i8b64", 4, 300, 8192),
    ("i8b32", 1, 3, 32), ("i8b32", 2, 70, 512), ("i8b32", 4, 130, 8192), ("i8b32", 7, 130, 2048),
    ("i8b32", 16, 64, 8192), ("i8b32", 11, 200, 5632), ("i8b32", 16, 1100, 1024), ("i8b32", 3, 20000, 1024),
]


@pytest.mark.parametrize("fmt,M,N,K", MULTI_SHAPES)
def test_multi_parity(oracle, fmt, M, N, K):
    say("gemv_multi", fmt, M, N, K)
    w, s = make(fmt, 2000 + N + K + M, N, K)
    if N > 3:
        w, s = set_scales(fmt, w, s, N, K, [2.0 ** -24, -0.75, 0.0, 3e-6])
    X = lqgen.activations(6000 + M + K, M * K, np.float16).reshape(M, K)
    Wd = gu.upload(fmt, w, s, N, K)
    Y = gu.gemv_multi(fmt, Wd, X, M, N, K)
    Yr, S = oracle.gemm(ORACLE_FMT[fmt], w, s, X, M, N, K)
    r = gu.ratio(Y, Yr, S, gu.GEMV_REL, gu.GEMV_ABS)
    assert r <= 1.0, f"tolerance ratio {r}"


@pytest.mark.parametrize("M", [16, 4, 2])
@pytest.mark.parametrize("fmt", ["q4_0", "q8_0", "i8b64", "i8b32"])
def test_multi_invariants(oracle, fmt, M):
    """Deterministic; doubling every scale doubles Y bit for bit; a one-hot
    token row gives the weight column exactly as lq_dequant_f32 unpacks it;
    each token row agrees with the single-token GEMV of that row."""
    N, K = 200, 2048 if fmt != "q4_0" else 896
    say("gemv_multi invariants", fmt, M, N, K)
    w, s = make(fmt, 4321, N, K)
    X = lqgen.activations(77, M * K, np.float16).reshape(M, K)
    Wd = gu.upload(fmt, w, s, N, K)
    Y1 = gu.gemv_multi(fmt, Wd, X, M, N, K)
    Y2 = gu.gemv_multi(fmt, Wd, X, M, N, K)
    assert np.array_equal(Y1.view(np.uint32), Y2.view(np.uint32)), "not deterministic"
    if fmt in gu.PLANAR:
        w2, s2 = w, s * np.float32(2)
    else:
        bb = 18 if fmt == "q4_0" else 34
        blk = w.reshape(-1, bb).copy()
        d = blk[:, 0:2].copy().view(np.float16) * np.float16(2)
        blk[:, 0:2] = d.view(np.uint8).reshape(-1, 2)
        w2, s2 = blk.reshape(-1), None
    Y3 = gu.gemv_multi(fmt, gu.upload(fmt, w2, s2, N, K), X, M, N, K)
    assert np.array_equal(Y3, 2 * Y1)
    out32 = torch.empty(N * K, dtype=torch.float32, device="cuda")
    lq.lq_dequant_f32(gu.FMT[fmt], Wd, out32, N, K)
    torch.cuda.synchronize()
    full = out32.cpu().numpy().reshape(N, K)
    ks = [0, 1, 15, 16, 31, 32, 63, 100, 257, 511, 640, K - 33, K - 17, K - 2, K - 1, 5]
    for j in range(0, len(ks), M):
        E = np.zeros((M, K), np.float16)
        for m, k in enumerate(ks[j:j + M]):
            E[m, k] = 1
        Ye = gu.gemv_multi(fmt, Wd, E, M, N, K)
        for m, k in enumerate(ks[j:j + M]):
            assert np.array_equal(Ye[m].view(np.uint32), full[:, k].view(np.uint32)), (m, k)
    for m in sorted({0, M // 2, M - 1}):
        y = gu.gemv(fmt, Wd, X[m], N, K)
        _, S = oracle.gemv(ORACLE_FMT[fmt], w, s, X[m], N, K)
        assert np.all(np.abs(Y1[m].astype(np.float64) - y) <= 2 * (gu.GEMV_REL * S + gu.GEMV_ABS)), m


@pytest.mark.parametrize("fmt,M,N,K", [("q4_0", 2, 151936 // 8, 896), ("q4_0", 2, 70, 25600),
                                        ("q8_0", 2, 8192, 2048), ("q8_0", 3, 130, 8192), ("q8_0", 4, 2048, 8192),
                                        ("i8b64", 2, 300, 5632), ("i8b64", 3, 2048, 8192), ("i8b64", 4, 70, 8192),
                                        ("i8b32", 3, 300, 4096), ("i8b32", 4, 20000, 1024)])
def test_few_tokens_equal_single_token_rows(fmt, M, N, K):
    """A few tokens share each weight load, but every token row goes through
    the arithmetic of lq_gemv with fp16 activations on the same K split: the
    rows are those GEMVs bit for bit (split and unsplit K)."""
    say("gemv_multi few tokens vs lq_gemv", fmt, M, N, K)
    w, s = make(fmt, 3300 + N + K, N, K)
    Wd = gu.upload(fmt, w, s, N, K)
    X = lqgen.activations(3400 + K + M, M * K, np.float16).reshape(M, K)
    Y = gu.gemv_multi(fmt, Wd, X, M, N, K)
    for m in range(M):
        y = gu.gemv(fmt, Wd, X[m], N, K)
        assert np.array_equal(Y[m].view(np.uint32), y.view(np.uint32)), m


def test_multi_zero_codes():
    """Q4_0 codes all 8 and Q8_0 / int8 codes all 0 give exactly zero."""
    M, N, K = 9, 100, 2048
    for fmt in ("q4_0", "q8_0", "i8b64", "i8b32"):
        say("gemv_multi zero codes", fmt)
        w, s = make(fmt, 5, N, K)
        if fmt in gu.PLANAR:
            w = np.zeros_like(w)
        else:
            bb = 18 if fmt == "q4_0" else 34
            blk = w.reshape(-1, bb).copy()
            blk[:, 2:] = 0x88 if fmt == "q4_0" else 0
            w = blk.reshape(-1)
        X = lqgen.activations(3, M * K, np.float16).reshape(M, K)
        Y = gu.gemv_multi(fmt, gu.upload(fmt, w, s, N, K), X, M, N, K)
        assert np.all(Y == 0)


def test_multi_batch_mixed(oracle):
    """Three formats, token counts 1..16, split and unsplit matrices, more
    descriptors than one launch holds: every output, grouped and alone,
    passes the oracle (the K split may differ between the two)."""
    cases = []
    for i in range(19):
        fmt = ["q4_0", "q8_0", "i8b64", "i8b32"][i % 4]
        K = [64, 896, 2048, 5632][i % 4] if fmt != "i8b64" else [64, 2048, 5632][i % 3]
        N = 11 + 53 * i
        M = 1 + (5 * i) % 16
        w, s = make(fmt, 800 + i, N, K)
        X = lqgen.activations(1900 + i, M * K, np.float16).reshape(M, K)
        cases.append((fmt, M, N, K, w, s, X))
    say("gemv_multi batch of", len(cases))
    descs, outs, devs = [], [], []
    for fmt, M, N, K, w, s, X in cases:
        Wd, Xd, Y = gu.upload(fmt, w, s, N, K), to_device(X), gu.guarded(M * N)
        devs.append((Wd, Xd))
        descs.append((gu.FMT[fmt], Wd, Xd, Y, M, N, K))
        outs.append(Y)
    lq.lq_gemv_multi_batch(descs, ws=gu.gemv_ws())
    torch.cuda.synchronize()
    for (fmt, M, N, K, w, s, X), Y, (Wd, Xd) in zip(cases, outs, devs):
        gu.check_guard(Y, M * N)
        got = Y[:M * N].cpu().numpy().reshape(M, N)
        Yr, S = oracle.gemm(ORACLE_FMT[fmt], w, s, X, M, N, K)
        assert gu.ratio(got, Yr, S, gu.GEMV_REL, gu.GEMV_ABS) <= 1.0, (fmt, M, N, K)
        single = gu.gemv_multi(fmt, Wd, X, M, N, K)
        assert gu.ratio(single, Yr, S, gu.GEMV_REL, gu.GEMV_ABS) <= 1.0, (fmt, M, N, K)


def test_matmul_routes_few_tokens_to_multi():
    """lq_matmul with 2..16 fp16 tokens is the multi-token GEMV, bit for bit."""
    N, K = 96, 512
    w, _ = make("q4_0", 12, N, K)
    Wd = gu.upload("q4_0", w, None, N, K)
    for M in (2, 9, 16):
        say("matmul routing", M)
        X = lqgen.activations(13 + M, M * K, np.float16).reshape(M, K)
        Ym = gu.gemv_multi("q4_0", Wd, X, M, N, K)
        Y = gu.guarded(M * N)
        lq.lq_matmul(lq.LQ_Q4_0, Wd, to_device(X), Y, M, N, K, ws=gu.gemv_ws())
        torch.cuda.synchronize()
        gu.check_guard(Y, M * N)
        assert np.array_equal(Y[:M * N].cpu().numpy().reshape(M, N), Ym), M


def test_multi_graph_replays_match_eager(oracle):
    """Split-K multi-token launches captured in a graph: every replay equals
    the eager result bit for bit, with eager runs in between."""
    say("gemv_multi graph replays")
    cases = [("q8_0", 16, 128, 4096), ("q4_0", 5, 64, 2048), ("i8b64", 3, 200, 5632)]
    data, outs = [], []
    for i, (fmt, M, N, K) in enumerate(cases):
        w, s = make(fmt, 7100 + i, N, K)
        X = lqgen.activations(7200 + i, M * K, np.float16).reshape(M, K)
        data.append((fmt, M, N, K, w, s, X, gu.upload(fmt, w, s, N, K), to_device(X)))
        outs.append(torch.zeros(M * N, device="cuda"))

    def run():
        for (fmt, M, N, K, _, _, _, Wd, Xd), Y in zip(data, outs):
            lq.lq_gemv_multi(gu.FMT[fmt], Wd, Xd, Y, M, N, K, ws=gu.gemv_ws())

    run()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    for (fmt, M, N, K, w, s, X, _, _), Y in zip(data, eager):
        Yr, S = oracle.gemm(ORACLE_FMT[fmt], w, s, X, M, N, K)
        assert gu.ratio(Y.cpu().numpy().reshape(M, N), Yr, S, gu.GEMV_REL, gu.GEMV_ABS) <= 1.0, fmt
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        run()
    for rep in range(3):
        for o in outs:
            o.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep} differs from the eager result"
        run()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"eager run after replay {rep} differs"


def _workload(oracle, wl, sample):
    M = wl.M
    worst = 0.0
    for m in wl.mats:
        say("gemv_multi workload", wl.name, m.name, M, m.N, m.K)
        w, s = m.generate()
        X = wl.x(m.xkey)
        Wd = gu.upload(m.fmt, w, s, m.N, m.K)
        Y = gu.gemv_multi(m.fmt, Wd, X, M, m.N, m.K)
        rng = np.random.default_rng(m.seed)
        ns = np.unique(np.concatenate([[0, 1, 63, 64, m.N - 2, m.N - 1], rng.integers(0, m.N, sample)]))
        Yr, S = oracle.gemm(ORACLE_FMT[m.fmt], w, s, X, M, m.N, m.K, ns=ns)
        r = gu.ratio(Y[:, ns], Yr, S, gu.GEMV_REL, gu.GEMV_ABS)
        assert r <= 1.0, (wl.name, m.name, r)
        worst = max(worst, r)
        del Wd
    return worst


@pytest.mark.slow
def test_workload_multi_lm_head(oracle):
    _workload(oracle, lqgen.multi_token(lqgen.q4_0_lmhead_151936x896(), 16), 2048)


@pytest.mark.slow
def test_workload_multi_q8_0_layer(oracle):
    _workload(oracle, lqgen.multi_token(lqgen.q8_0_layer_2048(0), 8), 1024)


@pytest.mark.slow
def test_workload_multi_i8b64_layer(oracle):
    _workload(oracle, lqgen.multi_token(lqgen.i8b64_tinyllama_layer(0), 4), 1024)


def _grouped_workload(oracle, wl, sample):
    """Every matrix of the workload in one lq_gemv_multi_batch call (the
    launch bench.py times), sampled rows of each against the oracle."""
    M = wl.M
    mats = [(m,) + tuple(m.generate()) for m in wl.mats]
    X = {k: wl.x(k) for k in wl.xs}
    Xd = {k: to_device(v) for k, v in X.items()}
    descs, outs, devs = [], [], []
    for m, w, s in mats:
        Wd, Y = gu.upload(m.fmt, w, s, m.N, m.K), gu.guarded(M * m.N)
        devs.append(Wd)
        descs.append((gu.FMT[m.fmt], Wd, Xd[m.xkey], Y, M, m.N, m.K))
        outs.append(Y)
    say("gemv_multi grouped workload", wl.name, M, len(mats))
    lq.lq_gemv_multi_batch(descs, ws=gu.gemv_ws())
    torch.cuda.synchronize()
    for (m, w, s), Y in zip(mats, outs):
        gu.check_guard(Y, M * m.N)
        got = Y[:M * m.N].cpu().numpy().reshape(M, m.N)
        rng = np.random.default_rng(m.seed + M)
        ns = np.unique(np.concatenate([[0, 1, 63, 64, m.N - 2, m.N - 1], rng.integers(0, m.N, sample)]))
        Yr, S = oracle.gemm(ORACLE_FMT[m.fmt], w, s, X[m.xkey], M, m.N, m.K, ns=ns)
        assert gu.ratio(got[:, ns], Yr, S, gu.GEMV_REL, gu.GEMV_ABS) <= 1.0, (wl.name, m.name, M)


@pytest.mark.slow
@pytest.mark.parametrize("M", [2, 4])
def test_workload_few_tokens_q8_0_layer_grouped(oracle, M):
    """The Q8_0 decoder layer at M = 2 and 4 in one grouped launch, as timed
    (few-token GEMV kernel, K split on the down projection)."""
    _grouped_workload(oracle, lqgen.multi_token(lqgen.q8_0_layer_2048(0), M), 1024)


@pytest.mark.slow
def test_workload_few_tokens_lm_head(oracle):
    """The Q4_0 LM head at M = 2 (few-token GEMV kernel), as timed."""
    wl = lqgen.multi_token(lqgen.q4_0_lmhead_151936x896(with_ffn=False), 2)
    _grouped_workload(oracle, wl, 4096)
