"""GPU parity of the activation-quantized integer-dot path (lq_quantize_act,
lq_gemv_q8act) against the CPU oracle.

The "oxinfer" page quantizes each matmul's activations and takes int8 dot
products with the weight codes ("How it works", quant.rs), with multi-token
variants for drafted tokens ("Speculative decoding").  Bars:
  * quantization: codes, scales and code sums bit-exact (both sides take the
    same fp32 steps);
  * product: per output |Y - Y_q| <= 1e-4 * sum_b |ws s I| + 1e-6 against the
    oracle's value of the same quantized product (the integer block sums are
    exact on both sides; only the fp32 scaling and accumulation round);
  * both kernels (vector dot products for few tokens, integer matrix cores
    for more) on every format;
  * exact case: unit weight scales and integer activations whose blocks reach
    127 (so s = 1 and q = x) make every term an integer; with K <= 1024 every
    partial sum is an integer below 2^24, so Y must equal the integer product
    exactly, whatever the summation order;
  * against the unquantized activations, the error stays within the
    quantization bound sum_b (s_b / 2) sum_k |w| plus the product's bar.
Every case prints its name before it touches the GPU.
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

Q8ACT_REL, Q8ACT_ABS = 1e-4, 1e-6


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    lq.load()
    lq.lq_init()
    yield


def quantize_gpu(X: np.ndarray, M, K):
    """lq_quantize_act on the device; returns (q, s, sum) on the host, after
    checking that nothing was written past any of the three outputs."""
    Xd = to_device(np.ascontiguousarray(X))
    nb = K // 32
    q = torch.full((M * K + 4096,), -77, dtype=torch.int8, device="cuda")
    s = gu.guarded(M * nb)
    t = torch.full((M * nb + gu.GUARD,), -999, dtype=torch.int32, device="cuda")
    lq.lq_quantize_act(Xd, M, K, q, s, t)
    torch.cuda.synchronize()
    assert torch.all(q[M * K:] == -77).item(), "write past the end of q"
    gu.check_guard(s, M * nb)
    assert torch.all(t[M * nb:] == -999).item(), "write past the end of sum"
    return (q[:M * K].cpu().numpy().reshape(M, K), s[:M * nb].cpu().numpy().reshape(M, nb),
            t[:M * nb].cpu().numpy().reshape(M, nb))


def q8act_gpu(fmt, Wd, q, s, t, M, N, K, ws=True):
    qd, sd, td = to_device(q), to_device(s), to_device(t)
    Y = gu.guarded(M * N)
    lq.lq_gemv_q8act(gu.FMT[fmt], Wd, qd, sd, td, Y, M, N, K, ws=gu.gemv_ws() if ws is True else ws)
    torch.cuda.synchronize()
    gu.check_guard(Y, M * N)
    return Y[:M * N].cpu().numpy().reshape(M, N)


def assert_quant_equal(got, want):
    for name, a, b in zip(("q", "s", "sum"), got, want):
        assert a.dtype == b.dtype and a.shape == b.shape, name
        assert np.array_equal(a.view(np.uint8) if a.dtype == np.float32 else a,
                              b.view(np.uint8) if b.dtype == np.float32 else b), name


# ---------------------------------------------------------- quantization ----

def special_rows(K, xdt):
    """Rows that exercise the rule's edges: a zero block, a block whose
    maximum is 127 with halves that round to even, a negative extreme, tiny
    and huge magnitudes (finite in the activation dtype)."""
    big, tiny = (1e30, 1e-30) if xdt == np.float32 else (1e3, 1e-6)
    rows = np.zeros((4, K), np.float32)
    nb = K // 32
    ties = np.array([127.0, 2.5, 3.5, -2.5, -0.5, 0.5, 126.5, -126.5, 1.5, -1.5, 4.5] + [0.25] * 21, np.float32)
    for b in range(nb):
        blk = slice(32 * b, 32 * b + 32)
        kind = b % 4
        if kind == 1:
            rows[0, blk] = ties
        elif kind == 2:
            rows[0, blk] = np.linspace(-0.4, 0.9, 32, dtype=np.float32)
            rows[0, 32 * b + 7] = -3.0
        elif kind == 3:
            rows[0, blk] = np.linspace(-1, 1, 32, dtype=np.float32) * np.float32(3e-38)
    rows[1] = lqgen.activations(77 + K, K, np.float32) * np.float32(big)
    rows[2] = lqgen.activations(78 + K, K, np.float32) * np.float32(tiny)
    rows[3] = np.round(lqgen.activations(79 + K, K, np.float32) * 40)
    return rows


QUANT_SHAPES = [(1, 32), (3, 96), (16, 896), (7, 5632), (2, 1 << 15), (300, 2048)]


@pytest.mark.parametrize("M,K", QUANT_SHAPES)
@pytest.mark.parametrize("xdt", [np.float32, np.float16], ids=["xf32", "xf16"])
def test_quantize_act_bitwise(oracle, M, K, xdt):
    say("quantize_act", M, K, np.dtype(xdt).name)
    X = lqgen.activations(9100 + M + K, M * K, np.float32).reshape(M, K)
    if M >= 4:
        X[:4] = special_rows(K, xdt)
    X = X.astype(xdt)
    assert np.all(np.isfinite(X))
    assert_quant_equal(quantize_gpu(X, M, K), oracle.quantize_act(X, M, K))


# --------------------------------------------------------------- product ----

# (fmt, M, N, K): every token count, ragged tiles (N % 64), one-block rows,
# K split across workgroups (few tiles, long rows), and many-tile launches.
Q8ACT_SHAPES = [
    ("q4_0", 1, 1, 32), ("q4_0", 2, 5, 64), ("q4_0", 3, 67, 96), ("q4_0", 16, 64, 896),
    ("q4_0", 5, 130, 960), ("q4_0", 8, 300, 2048), ("q4_0", 13, 33, 11008), ("q4_0", 16, 2500, 896),
    ("q4_0", 4, 17, 25600), ("q4_0", 1, 3000, 640),
    ("q8_0", 1, 3, 32), ("q8_0", 2, 70, 512), ("q8_0", 7, 130, 2048), ("q8_0", 16, 64, 8192),
    ("q8_0", 11, 200, 5632), ("q8_0", 1, 8200, 1024),
    ("i8b64", 1, 1, 64), ("i8b64", 3, 77, 128), ("i8b64", 16, 256, 2048), ("i8b64", 6, 45, 5632),
    ("i8b64", 16, 130, 8192), ("i8b64", 9, 5, 30720), ("i8b64", 1, 1500, 512),
    ("i8b32", 1, 3, 32), ("i8b32", 2, 70, 512), ("i8b32", 4, 130, 8192), ("i8b32", 15, 1100, 1024),
    ("i8b32", 12, 20000, 256),
    # the matrix-core kernel (Q4_0 from 7 tokens, the int8 formats at 16):
    # partial tiles, K split, one-block rows
    ("q4_0", 7, 1, 32), ("q4_0", 7, 200, 4096), ("q4_0", 11, 64, 25600), ("q4_0", 16, 3000, 640),
    ("q8_0", 16, 100, 2048), ("q8_0", 16, 3, 32), ("i8b64", 16, 1, 64), ("i8b32", 16, 300, 1024),
    ("i8b32", 16, 5, 30720),
]


@pytest.mark.parametrize("fmt,M,N,K", Q8ACT_SHAPES)
def test_q8act_parity(oracle, fmt, M, N, K):
    say("gemv_q8act", fmt, M, N, K)
    w, s = make(fmt, 3000 + N + K + M, N, K)
    if N > 3:
        w, s = set_scales(fmt, w, s, N, K, [2.0 ** -24, -0.75, 0.0, 3e-6])
    X = lqgen.activations(7000 + M + K, M * K, np.float32).reshape(M, K)
    qa = quantize_gpu(X, M, K)
    qr = oracle.quantize_act(X, M, K)
    assert_quant_equal(qa, qr)
    Wd = gu.upload(fmt, w, s, N, K)
    Y = q8act_gpu(fmt, Wd, *qa, M, N, K)
    Yr, S = oracle.gemv_q8act(ORACLE_FMT[fmt], w, s, qr[0], qr[1], M, N, K)
    r = gu.ratio(Y, Yr, S, Q8ACT_REL, Q8ACT_ABS)
    assert r <= 1.0, f"tolerance ratio {r}"
    if fmt == "i8b32" or N < 64:
        # without a workspace every tile keeps its K in one workgroup
        Y1 = q8act_gpu(fmt, Wd, *qa, M, N, K, ws=None)
        r = gu.ratio(Y1, Yr, S, Q8ACT_REL, Q8ACT_ABS)
        assert r <= 1.0, f"tolerance ratio without workspace {r}"


def unit_scale_weights(fmt, seed, N, K):
    """Generated codes with every block scale set to 1."""
    w, s = make(fmt, seed, N, K)
    if fmt in gu.PLANAR:
        return w, np.ones_like(s)
    bb = 18 if fmt == "q4_0" else 34
    blk = w.reshape(-1, bb).copy()
    blk[:, 0:2] = np.array([1.0], np.float16).view(np.uint8)
    return blk.reshape(-1), None


@pytest.mark.parametrize("fmt,M,N,K", [("q4_0", 5, 130, 1024), ("q8_0", 16, 70, 1024),
                                       ("i8b64", 3, 200, 1024), ("i8b32", 16, 64, 512),
                                       ("q4_0", 1, 17, 1024), ("q8_0", 9, 1, 992),
                                       ("q4_0", 9, 70, 1024), ("i8b64", 16, 130, 1024)])
def test_q8act_exact_integers(oracle, fmt, M, N, K):
    say("gemv_q8act exact integers", fmt, M, N, K)
    w, s = unit_scale_weights(fmt, 4100 + N, N, K)
    rng_codes = np.round(lqgen.activations(4200 + K + M, M * K, np.float32) * 45).clip(-127, 127)
    X = rng_codes.reshape(M, K).astype(np.float32)
    X[:, ::32] = 127.0                       # every block's maximum is 127: s = 1, q = X
    q, sc, t = quantize_gpu(X, M, K)
    assert np.all(sc == 1.0) and np.array_equal(q.astype(np.float32), X)
    Wq = oracle.dequant(ORACLE_FMT[fmt], w, s, N, K)       # exact integer codes (scale 1)
    assert np.abs(Wq).sum(axis=1).max() * 127 < 2 ** 24
    want = (X.astype(np.float64) @ Wq.T)
    Wd = gu.upload(fmt, w, s, N, K)
    Y = q8act_gpu(fmt, Wd, q, sc, t, M, N, K)
    assert np.array_equal(Y.astype(np.float64), want)


@pytest.mark.parametrize("fmt,M,N,K", [("q4_0", 4, 130, 960), ("q8_0", 16, 70, 2048),
                                       ("i8b64", 7, 64, 1024), ("i8b32", 2, 33, 4096)])
def test_q8act_quantization_error_bound(oracle, fmt, M, N, K):
    """Against the unquantized activations: |Y - W x| <= sum_k |w_k| s_b / 2
    (each activation moves by at most half its block's step) plus the
    product's own bar."""
    say("gemv_q8act error bound", fmt, M, N, K)
    w, s = make(fmt, 5100 + N + K, N, K)
    X = lqgen.activations(5200 + M + K, M * K, np.float32).reshape(M, K)
    q, sc, t = quantize_gpu(X, M, K)
    Wd = gu.upload(fmt, w, s, N, K)
    Y = q8act_gpu(fmt, Wd, q, sc, t, M, N, K)
    Wf = oracle.dequant(ORACLE_FMT[fmt], w, s, N, K)
    half_step = np.repeat(sc.astype(np.float64) / 2, 32, axis=1)          # M x K
    bound = half_step @ np.abs(Wf).T                                       # M x N
    _, Sq = oracle.gemv_q8act(ORACLE_FMT[fmt], w, s, q, sc, M, N, K)
    for m in range(M):
        y, _ = oracle.gemv(ORACLE_FMT[fmt], w, s, X[m], N, K)
        err = np.abs(Y[m].astype(np.float64) - y)
        lim = bound[m] * (1 + 1e-6) + Q8ACT_REL * Sq[m] + Q8ACT_ABS
        assert np.all(err <= lim), float(np.max(err / lim))
    # the bound is not vacuous: quantization moves the result visibly
    y0, _ = oracle.gemv(ORACLE_FMT[fmt], w, s, X[0], N, K)
    assert np.max(np.abs(Y[0] - y0)) > 0


# --------------------------------------------------------- full size ----

def _rows_of(fmt, w, s, N, K, rows):
    """The selected rows of a generated matrix, as a matrix of their own."""
    rows = np.asarray(rows)
    if fmt in gu.PLANAR:
        E = 64 if fmt == "i8b64" else 32
        return w.reshape(N, K)[rows].reshape(-1), s.reshape(N, K // E)[rows].reshape(-1)
    return w.reshape(N, -1)[rows].reshape(-1), None


@pytest.mark.slow
@pytest.mark.parametrize("M", [1, 16])
def test_q8act_lm_head_full_size(oracle, M):
    """Q4_0 LM head 151936 x 896 at M tokens, in the launch configuration the
    benchmark times (workspace given): the quantized activations bit-exact,
    4,096 sampled rows (first and last tiles included) against the oracle."""
    say("gemv_q8act LM head 151936x896 M", M)
    wl = lqgen.q4_0_lmhead_151936x896(with_ffn=False)
    mat = wl.mats[0]
    N, K = mat.N, mat.K
    w, s = mat.generate()
    seed, n, _ = wl.xs["x"]
    X = lqgen.activations(seed, M * n, np.float32).reshape(M, n)
    qa = quantize_gpu(X, M, K)
    qr = oracle.quantize_act(X, M, K)
    assert_quant_equal(qa, qr)
    Wd = gu.upload("q4_0", w, s, N, K)
    Y = q8act_gpu("q4_0", Wd, *qa, M, N, K)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(N - 64, N),
                                     rng.choice(N, 4096 - 128, replace=False)]))
    ws_, ss_ = _rows_of("q4_0", w, s, N, K, rows)
    Yr, S = oracle.gemv_q8act(ORACLE_FMT["q4_0"], ws_, ss_, qr[0], qr[1], M, len(rows), K)
    r = gu.ratio(Y[:, rows], Yr, S, Q8ACT_REL, Q8ACT_ABS)
    assert r <= 1.0, f"tolerance ratio {r}"


def test_q8act_graph_replays_and_two_streams(oracle):
    """Quantization plus both product kernels, with K split across
    workgroups (few tiles, long rows), captured in one graph and replayed
    several times with eager runs in between: every replay equals the eager
    result bit for bit.  Then the same work on two streams at once, each
    with its own workspace, gives the same bits."""
    say("gemv_q8act graph replays and two streams")
    cases = [("q4_0", 3, 96, 11008), ("q4_0", 12, 130, 4096), ("q8_0", 16, 64, 8192), ("i8b64", 2, 200, 5632)]
    bufs = []
    for i, (fmt, M, N, K) in enumerate(cases):
        w, s = make(fmt, 3600 + i, N, K)
        X = lqgen.activations(3700 + i, M * K, np.float32).reshape(M, K)
        Xd = to_device(X)
        q = torch.empty(M * K, dtype=torch.int8, device="cuda")
        sc = torch.empty(M * K // 32, dtype=torch.float32, device="cuda")
        t = torch.empty(M * K // 32, dtype=torch.int32, device="cuda")
        Y = torch.zeros(M * N, device="cuda")
        bufs.append((fmt, M, N, K, w, s, X, Xd, gu.upload(fmt, w, s, N, K), q, sc, t, Y))

    def run(ws, sel=None):
        for fmt, M, N, K, _, _, _, Xd, Wd, q, sc, t, Y in (bufs if sel is None else sel):
            lq.lq_quantize_act(Xd, M, K, q, sc, t)
            lq.lq_gemv_q8act(gu.FMT[fmt], Wd, q, sc, t, Y, M, N, K, ws=ws)

    run(gu.gemv_ws())
    torch.cuda.synchronize()
    eager = [b[-1].clone() for b in bufs]
    for (fmt, M, N, K, w, s, X, *_), y in zip(bufs, eager):
        qr, sr, _ = oracle.quantize_act(X, M, K)
        Yr, S = oracle.gemv_q8act(ORACLE_FMT[fmt], w, s, qr, sr, M, N, K)
        assert gu.ratio(y.cpu().numpy().reshape(M, N), Yr, S, Q8ACT_REL, Q8ACT_ABS) <= 1.0, fmt
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        run(gu.gemv_ws())
    for rep in range(3):
        for b in bufs:
            b[-1].fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for b, e in zip(bufs, eager):
            assert torch.equal(b[-1], e), f"replay {rep} differs from the eager result ({b[0]}, M={b[1]})"
        run(gu.gemv_ws())
        torch.cuda.synchronize()
        for b, e in zip(bufs, eager):
            assert torch.equal(b[-1], e), f"eager run after replay {rep} differs"
    # two streams at once, each with its own workspace
    for b in bufs:
        b[-1].fill_(-1.0)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        run(gu.gemv_ws(1), bufs[0::2])
    with torch.cuda.stream(s2):
        run(gu.gemv_ws(2), bufs[1::2])
    torch.cuda.synchronize()
    for b, e in zip(bufs, eager):
        assert torch.equal(b[-1], e), f"two-stream run differs ({b[0]}, M={b[1]})"
