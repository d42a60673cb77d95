"""GPU checks of the boundary's contract beyond plain parity (needs an MI355X):
GEMV workspaces (none, garbage-filled, shared with a GEMM, one per stream on
two streams at once), non-finite scales, routing by token count, and a GEMM
whose activations exceed 4 GiB.  Expected values come only from the oracle.
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


# Shapes whose launches split K across workgroups when a workspace is given
# (few 64-row tiles, long rows), one per format.
SPLIT_CASES = [("q8_0", 2048, 8192, np.float32), ("q4_0", 96, 11008, np.float16),
               ("i8b64", 300, 5632, np.float16), ("i8b32", 128, 4096, np.float32)]


def _case(i, fmt, N, K, xdt):
    w, s = make(fmt, 9100 + i, N, K)
    x = lqgen.activations(9200 + i, K, xdt)
    return w, s, x, gu.upload(fmt, w, s, N, K)


@pytest.mark.parametrize("idx", range(len(SPLIT_CASES)))
def test_gemv_without_workspace(oracle, idx):
    """No workspace: every tile's K stays in one workgroup; still at the GEMV bar."""
    fmt, N, K, xdt = SPLIT_CASES[idx]
    say("gemv without workspace", fmt, N, K)
    w, s, x, Wd = _case(idx, fmt, N, K, xdt)
    y = gu.gemv(fmt, Wd, x, N, K, ws=None)
    yr, S = oracle.gemv(ORACLE_FMT[fmt], w, s, x, N, K)
    assert gu.ratio(y, yr, S, gu.GEMV_REL, gu.GEMV_ABS) <= 1.0


def test_gemv_workspace_shared_with_gemm(oracle):
    """A workspace that a split-K GEMM has just filled with its partial sums,
    then a GEMV on the same stream: the GEMV reads no leftover as an arrival."""
    fmt, N, K, xdt = SPLIT_CASES[0]
    say("gemv workspace after a gemm", fmt, N, K)
    w, s, x, Wd = _case(0, fmt, N, K, xdt)
    Mg, Ng, Kg = 64, 256, 4096
    wg, _ = make("q4_0", 9300, Ng, Kg)
    Wg = gu.upload("q4_0", wg, None, Ng, Kg)
    Xg = to_device(lqgen.activations(9301, Mg * Kg, np.float16).reshape(Mg, Kg))
    need = lq.lq_gemm_workspace_bytes(lq.LQ_Q4_0, Mg, Ng, Kg)
    assert need > 0
    ws = torch.empty(max(need, lq.lq_gemv_workspace_bytes()), dtype=torch.uint8, device="cuda")
    Yg = torch.empty(Mg * Ng, device="cuda")
    want = gu.gemv(fmt, Wd, x, N, K)          # same launch plan, the shared workspace
    for rep in range(3):
        lq.lq_gemm(lq.LQ_Q4_0, Wg, Xg, Yg, Mg, Ng, Kg, ws=ws)
        y = gu.guarded(N)
        lq.lq_gemv(gu.FMT[fmt], Wd, to_device(x), y, N, K, ws=ws)
        torch.cuda.synchronize()
        gu.check_guard(y, N)
        assert np.array_equal(y[:N].cpu().numpy(), want), rep
    yr, S = oracle.gemv(ORACLE_FMT[fmt], w, s, x, N, K)
    assert gu.ratio(want, yr, S, gu.GEMV_REL, gu.GEMV_ABS) <= 1.0


def test_gemv_two_streams(oracle):
    """Split-K GEMVs enqueued on two streams (same priority) that run at the
    same time, each with its own workspace, many launches each: every result
    equals the one-stream result bit for bit, and that passes the oracle."""
    say("gemv on two streams at once")
    data = [_case(i, *c) for i, c in enumerate(SPLIT_CASES)]
    want = []
    for (fmt, N, K, _), (w, s, x, Wd) in zip(SPLIT_CASES, data):
        y = gu.gemv(fmt, Wd, x, N, K)
        yr, S = oracle.gemv(ORACLE_FMT[fmt], w, s, x, N, K)
        assert gu.ratio(y, yr, S, gu.GEMV_REL, gu.GEMV_ABS) <= 1.0, fmt
        want.append(y)
    xs = [to_device(x) for (_, _, x, _) in data]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [gu.gemv_ws(1), gu.gemv_ws(2)]
    reps = 40
    # outs[stream][rep][case]
    outs = [[[torch.empty(c[1], device="cuda") for c in SPLIT_CASES] for _ in range(reps)] for _ in streams]
    torch.cuda.synchronize()
    for rep in range(reps):
        for si, st in enumerate(streams):
            descs = [(gu.FMT[c[0]], d[3], xs[i], outs[si][rep][i], c[1], c[2])
                     for i, (c, d) in enumerate(zip(SPLIT_CASES, data))]
            # one launch per matrix, so each stream keeps several split launches in flight
            for dsc in descs:
                lq.lq_gemv_batch([dsc], ws=wss[si], stream=st)
    torch.cuda.synchronize()
    for si in range(len(streams)):
        for rep in range(reps):
            for i, c in enumerate(SPLIT_CASES):
                got = outs[si][rep][i].cpu().numpy()
                assert np.array_equal(got, want[i]), (si, rep, c[0])


def _nonfinite_matrix(fmt, N, K, seed):
    """A matrix with special scales in chosen rows, and the row sets they
    decide.  Block `b` of rows 0-5 gets a NaN scale; of rows 6-11 +inf and
    of rows 12-17 -inf, with codes whose weights are all positive there
    (x is positive on that block), so the exact sum is +inf / -inf; rows 18-23
    get +inf with mixed-sign codes.  The last block of rows 24-29 gets +inf
    with positive weights too (the last unit of the last wave: a batch slot
    past it re-reads it and must not touch the sum)."""
    w, s = make(fmt, seed, N, K)
    E = 64 if fmt == "i8b64" else 32
    nb = K // E
    b = 3
    plan = [(range(0, 6), b, np.nan, False), (range(6, 12), b, np.inf, True),
            (range(12, 18), b, -np.inf, True), (range(18, 24), b, np.inf, False),
            (range(24, 30), nb - 1, np.inf, True)]
    if fmt in gu.PLANAR:
        codes = w.reshape(N, K).copy()
        sc = s.reshape(N, nb).copy()
        for rows, blk, val, pos in plan:
            for r in rows:
                sc[r, blk] = val
                if pos:
                    codes[r, blk * E:(blk + 1) * E] = np.abs(codes[r, blk * E:(blk + 1) * E]) % 127 + 1
        return codes.reshape(-1), sc.reshape(-1), plan
    bb = 18 if fmt == "q4_0" else 34
    blk_bytes = w.reshape(N, nb, bb).copy()
    for rows, blk, val, pos in plan:
        for r in rows:
            blk_bytes[r, blk, 0:2] = np.array([val], np.float64).astype(np.float16).view(np.uint8)
            if pos:
                if fmt == "q4_0":   # codes 9..15 in both nibbles: q - 8 > 0
                    c = blk_bytes[r, blk, 2:]
                    blk_bytes[r, blk, 2:] = (((c & 0x7) | 0x9) & 0xF) | ((((c >> 4) & 0x7) | 0x9) << 4)
                else:
                    c = blk_bytes[r, blk, 2:].view(np.int8)
                    blk_bytes[r, blk, 2:] = (np.abs(c.astype(np.int16)) % 127 + 1).astype(np.uint8)
    return blk_bytes.reshape(-1), None, plan


def _positive_blocks(v, plan, E, axis_len):
    v = v.copy()
    for _, blk, _, pos in plan:
        if pos:
            sl = (Ellipsis, slice(blk * E, (blk + 1) * E))
            v[sl] = np.abs(v[sl]) + np.float16(0.25).astype(v.dtype)
    return v


def _check_nonfinite(y, yr, S, plan, what):
    """Finite oracle rows at the bar; +-inf oracle rows equal, sign and all;
    NaN oracle rows non-finite; NaN-scale rows NaN."""
    y = np.asarray(y, np.float64)
    fin = np.isfinite(yr)
    assert np.all(np.isfinite(y[fin])), what
    assert gu.ratio(y[fin], yr[fin], S[fin], *what[1]) <= 1.0, what
    inf = np.isinf(yr)
    assert inf.sum() > 0, what
    assert np.array_equal(y[inf], yr[inf]), what
    nanr = np.isnan(yr)
    assert np.all(~np.isfinite(y[nanr])), what
    rows = np.array(list(plan[0][0]))
    assert np.all(np.isnan(y[..., rows])), what


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0", "i8b64", "i8b32"])
def test_nonfinite_scales(oracle, fmt):
    """A NaN scale makes its rows NaN; an infinite scale makes them
    non-finite, and exactly +-inf where every product it scales has one
    sign (then the exact sum is that infinity): single-token GEMV (fp32 and
    fp16 x, with and without a workspace), multi-token GEMV (M = 3 and 8)
    and the GEMM."""
    E = 64 if fmt == "i8b64" else 32
    for K in (2048, 1344 if fmt == "i8b64" else 960):
        N = 130
        say("non-finite scales", fmt, N, K)
        w, s, plan = _nonfinite_matrix(fmt, N, K, 9500 + K)
        Wd = gu.upload(fmt, w, s, N, K)
        for xdt in (np.float32, np.float16):
            x = _positive_blocks(lqgen.activations(9600 + K, K, xdt), plan, E, K)
            yr, S = oracle.gemv(ORACLE_FMT[fmt], w, s, x, N, K)
            for ws in (True, None):
                y = gu.gemv(fmt, Wd, x, N, K, ws=ws)
                _check_nonfinite(y, yr, S, plan, ("gemv", (gu.GEMV_REL, gu.GEMV_ABS), fmt, K, xdt, ws))
        for M in (3, 8):
            X = _positive_blocks(lqgen.activations(9700 + K + M, M * K, np.float16).reshape(M, K), plan, E, K)
            Yr, S = oracle.gemm(ORACLE_FMT[fmt], w, s, X, M, N, K)
            Y = gu.gemv_multi(fmt, Wd, X, M, N, K)
            _check_nonfinite(Y, Yr, S, plan, ("gemv_multi", (gu.GEMV_REL, gu.GEMV_ABS), fmt, K, M))
        M = 40
        X = _positive_blocks(lqgen.activations(9800 + K, M * K, np.float16).reshape(M, K), plan, E, K)
        Yr, S = oracle.gemm(ORACLE_FMT[fmt], w, s, X, M, N, K)
        Y = gu.gemm(Wd, X, M, N, K, fmt)
        _check_nonfinite(Y, Yr, S, plan, ("gemm", (gu.GEMM_REL, gu.GEMM_ABS), fmt, K))


@pytest.mark.parametrize("M", [16, 17, 512])
def test_matmul_threshold(oracle, M):
    """lq_matmul at the edges of its routing: 16 tokens run the multi-token
    GEMV (bit for bit) at the GEMV bar, 17 and 512 the tile GEMM (bit for
    bit) at the GEMM bar."""
    N, K = 320, 1024
    say("matmul threshold", M, N, K)
    w, _ = make("q4_0", 9900 + M, N, K)
    Wd = gu.upload("q4_0", w, None, N, K)
    X = lqgen.activations(9901 + M, M * K, np.float16).reshape(M, K)
    need = max(lq.lq_gemm_workspace_bytes(lq.LQ_Q4_0, M, N, K), lq.lq_gemv_workspace_bytes())
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    Y = gu.guarded(M * N)
    lq.lq_matmul(lq.LQ_Q4_0, Wd, to_device(X), Y, M, N, K, ws=ws)
    torch.cuda.synchronize()
    gu.check_guard(Y, M * N)
    Y = Y[:M * N].cpu().numpy().reshape(M, N)
    Yr, S = oracle.gemm(0, w, None, X, M, N, K)
    if M <= 16:
        assert np.array_equal(Y, gu.gemv_multi("q4_0", Wd, X, M, N, K))
        assert gu.ratio(Y, Yr, S, gu.GEMV_REL, gu.GEMV_ABS) <= 1.0
    else:
        assert np.array_equal(Y, gu.gemm(Wd, X, M, N, K))
        assert gu.ratio(Y, Yr, S, gu.GEMM_REL, gu.GEMM_ABS) <= 1.0


@pytest.mark.slow
def test_gemm_x_above_4gib(oracle):
    """X of 4 GiB and more (M K 2 bytes >= 2^32): rows on both sides of the
    2 GiB and 4 GiB byte offsets, and the last row, against the oracle."""
    M, N, K = (1 << 20) + 37, 64, 2048
    say("gemm X above 4 GiB", M, N, K)
    w, _ = make("q4_0", 9950, N, K)
    Wd = gu.upload("q4_0", w, None, N, K)
    g = torch.Generator(device="cuda")
    g.manual_seed(9951)
    Xd = torch.randn(M * K, generator=g, device="cuda", dtype=torch.float16)
    assert Xd.numel() * 2 >= 1 << 32
    need = lq.lq_gemm_workspace_bytes(lq.LQ_Q4_0, M, N, K)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    Y = torch.empty(M * N, device="cuda")
    lq.lq_gemm(lq.LQ_Q4_0, Wd, Xd, Y, M, N, K, ws=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9952)
    rows = np.unique(np.concatenate([[0, 1, 524287, 524288, 1048575, 1048576, 1048577, M - 1],
                                     rng.integers(0, M, 24)]))
    idx = torch.from_numpy(rows).to("cuda")
    Xs = Xd.view(M, K).index_select(0, idx).cpu().numpy()
    Ys = Y.view(M, N).index_select(0, idx).cpu().numpy()
    del Xd, Y
    torch.cuda.empty_cache()
    Yr, S = oracle.gemm(0, w, None, Xs, len(rows), N, K)
    assert gu.ratio(Ys, Yr, S, gu.GEMM_REL, gu.GEMM_ABS) <= 1.0
