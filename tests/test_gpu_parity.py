"""GPU parity of liblq against the CPU oracle (needs an MI355X).

Every case prints its name before it touches the GPU.  Inputs come from the
seeded generator; expected values come only from the oracle or from the
hand-built blocks.  Bars: unpacked weights bit-exact; GEMV per row
|y - y_ref| <= 1e-4 * sum|w x| + 1e-6; GEMM per element
|Y - Y_ref| <= 2e-3 * sum|w x| + 1e-5.
"""
import json
import os
import sys

import numpy as np
import pytest
import torch

import gemm_q4_q8_int8_amd as lq
import lqgen
from gemm_q4_q8_int8_amd.device import to_device, upload_planes
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

ORACLE_FMT = {"q4_0": 0, "q8_0": 1, "i8b64": 2, "i8b32": 3}


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    lq.load()
    lq.lq_init()
    yield


def make(fmt, seed, N, K, c=None):
    if fmt == "q4_0":
        return lqgen.q4_0_aos(seed, N, K, c or 0.02), None
    if fmt == "q8_0":
        return lqgen.q8_0_aos(seed, N, K, c or 0.005), None
    return lqgen.i8_planes(seed, N, K, 64 if fmt == "i8b64" else 32, c or 0.003)


def set_scales(fmt, w, scales, N, K, values):
    """Overwrite the first scales of a generated matrix with special values."""
    if fmt in gu.PLANAR:
        s = scales.copy()
        s[:len(values)] = np.array(values, np.float32)
        return w, s
    bb = 18 if fmt == "q4_0" else 34
    blk = w.reshape(-1, bb).copy()
    for i, v in enumerate(values):
        blk[i, 0:2] = np.array([v], np.float64).astype(np.float16).view(np.uint8)
    return blk.reshape(-1), None


def ref_dequant(o, fmt, w, scales, N, K):
    return o.dequant_f32(ORACLE_FMT[fmt], w, scales, N, K), o.dequant_f16(ORACLE_FMT[fmt], w, scales, N, K)


# ------------------------------------------------------------- dequant ----

@pytest.mark.parametrize("fmt", ["q4_0", "q8_0", "i8b64", "i8b32"])
def test_dequant_bitwise(oracle, fmt):
    N, K = 37, 448 if fmt != "i8b64" else 448
    say("dequant", fmt, N, K)
    w, s = make(fmt, 101, N, K)
    specials = [2.0 ** -24, -2.0 ** -24, 3 * 2.0 ** -20, -0.0, 0.0, -1.5, 65504.0, np.inf, -np.inf, np.nan,
                6.1e-5, 1e-7]
    w, s = set_scales(fmt, w, s, N, K, specials)
    Wd = gu.upload(fmt, w, s, N, K)
    out32 = torch.empty(N * K, dtype=torch.float32, device="cuda")
    out16 = torch.empty(N * K, dtype=torch.uint16, device="cuda")
    lq.lq_dequant_f32(gu.FMT[fmt], Wd, out32, N, K)
    lq.lq_dequant_f16(gu.FMT[fmt], Wd, out16, N, K)
    torch.cuda.synchronize()
    g32 = out32.cpu().numpy().reshape(N, K)
    g16 = out16.cpu().numpy().reshape(N, K)
    r32, r16 = ref_dequant(oracle, fmt, w, s, N, K)
    nan = np.isnan(r32)
    assert np.array_equal(np.isnan(g32), nan)
    assert np.array_equal(g32.view(np.uint32)[~nan], r32.view(np.uint32)[~nan])
    n16 = np.isnan(r16.view(np.float16))
    assert np.array_equal(np.isnan(g16.view(np.float16)), n16)
    assert np.array_equal(g16[~n16], r16[~n16])


def test_dequant_golden_blocks(oracle):
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "blocks.json")))
    for blk in gold["blocks"]:
        say("golden block", blk["id"])
        raw = np.frombuffer(bytes.fromhex(blk["hex"]), np.uint8).copy()
        Wd = gu.upload(blk["fmt"], raw, None, 1, 32)
        out32 = torch.empty(32, dtype=torch.float32, device="cuda")
        out16 = torch.empty(32, dtype=torch.uint16, device="cuda")
        lq.lq_dequant_f32(gu.FMT[blk["fmt"]], Wd, out32, 1, 32)
        lq.lq_dequant_f16(gu.FMT[blk["fmt"]], Wd, out16, 1, 32)
        torch.cuda.synchronize()
        want = np.array([float(v) for v in blk["expected"]]).astype(np.float32)
        assert np.array_equal(out32.cpu().numpy().view(np.uint32), want.view(np.uint32)), blk["id"]
        want16 = np.array([float(v) for v in blk.get("f16", blk["expected"])]).astype(np.float16)
        assert np.array_equal(out16.cpu().numpy(), want16.view(np.uint16)), blk["id"]
        y = gu.gemv(blk["fmt"], Wd, np.ones(32, np.float32), 1, 32)
        if np.isfinite(float(blk["sum"])) and abs(float(blk["sum"])) < 1e6:
            assert y[0] == np.float32(float(blk["sum"])), blk["id"]


@pytest.mark.parametrize("N", [9, 64, 130])
def test_repack_roundtrip_planes(N):
    """lq_repack_gguf and lq_pack_planes both produce the documented tiled
    layout, byte for byte, as built on the host from the same blocks."""
    for fmt in ("q4_0", "q8_0", "i8b64", "i8b32"):
        K = 128 if fmt == "i8b64" else 224
        say("packed layout", fmt, N, K)
        w, s = make(fmt, 77 + N, N, K)
        if fmt in gu.PLANAR:
            E = 64 if fmt == "i8b64" else 32
            codes = w.reshape(N, K // E, E)
            scales = s.reshape(N, K // E)
        else:
            bb = 18 if fmt == "q4_0" else 34
            blk = w.view(np.uint8).reshape(N, K // 32, bb)
            codes = np.ascontiguousarray(blk[:, :, 2:])
            scales = np.ascontiguousarray(blk[:, :, 0:2]).view(np.uint16).reshape(N, K // 32)
        want = gu.tiled_reference(fmt, codes, scales, N, K)
        cb = N * K // 2 if fmt == "q4_0" else N * K
        off = lq.lq_scale_offset(gu.FMT[fmt], N, K)
        got = [("pack_planes", upload_planes(gu.FMT[fmt], codes.reshape(-1), scales.reshape(-1), N, K))]
        if fmt not in gu.PLANAR:
            got.append(("repack_gguf", gu.upload(fmt, w, None, N, K)))
        for name, Wd in got:
            b = Wd.cpu().numpy()
            assert b.size == want.size, name
            # the bytes between the planes are padding and left as allocated
            assert np.array_equal(b[:cb], want[:cb]), name + " codes"
            assert np.array_equal(b[off:], want[off:]), name + " scales"


# ---------------------------------------------------------------- GEMV ----

GEMV_SHAPES = [
    ("q4_0", 1, 32), ("q4_0", 5, 64), ("q4_0", 67, 96), ("q4_0", 300, 896), ("q4_0", 129, 960),
    ("q4_0", 33, 2048), ("q4_0", 40, 4864), ("q4_0", 17, 11008), ("q4_0", 9, 25600),
    ("q8_0", 1, 32), ("q8_0", 70, 512), ("q8_0", 130, 2048), ("q8_0", 31, 5632), ("q8_0", 24, 8192),
    ("q8_0", 6, 26624),
    ("i8b64", 1, 64), ("i8b64", 77, 128), ("i8b64", 256, 2048), ("i8b64", 45, 5632),
    ("i8b64", 12, 8192), ("i8b64", 5, 30720),
    ("i8b32", 1, 32), ("i8b32", 77, 96), ("i8b32", 256, 2048), ("i8b32", 45, 5632), ("i8b32", 5, 30720),
    ("i8b32", 20000, 1024),
]


@pytest.mark.parametrize("fmt,N,K", GEMV_SHAPES)
@pytest.mark.parametrize("xdt", [np.float32, np.float16], ids=["xf32", "xf16"])
def test_gemv_parity(oracle, fmt, N, K, xdt):
    say("gemv", fmt, N, K, np.dtype(xdt).name)
    w, s = make(fmt, 1000 + N + K, N, K)
    if N > 3:
        w, s = set_scales(fmt, w, s, N, K, [2.0 ** -24, -0.75, 0.0, 3e-6])
    x = lqgen.activations(4242 + K, K, xdt)
    Wd = gu.upload(fmt, w, s, N, K)
    y = gu.gemv(fmt, Wd, x, N, K)
    yr, S = oracle.gemv(ORACLE_FMT[fmt], w, s, x, N, K)
    r = gu.ratio(y, yr, S, gu.GEMV_REL, gu.GEMV_ABS)
    assert r <= 1.0, f"tolerance ratio {r}"


def test_gemv_batch_mixed(oracle):
    """More than one launch group and more descriptors than one launch holds."""
    cases = []
    for i in range(24):
        fmt = ["q4_0", "q8_0", "i8b64", "i8b32"][i % 4]
        K = [64, 896, 2048, 5632][i % 4] if fmt != "i8b64" else [64, 2048, 5632][i % 3]
        N = 13 + 37 * i
        xdt = np.float16 if i % 2 else np.float32
        w, s = make(fmt, 500 + i, N, K)
        x = lqgen.activations(900 + i, K, xdt)
        cases.append((fmt, N, K, w, s, x))
    say("gemv batch of", len(cases))
    descs, outs = [], []
    for fmt, N, K, w, s, x in cases:
        Wd = gu.upload(fmt, w, s, N, K)
        xd = to_device(x)
        y = gu.guarded(N)
        descs.append((gu.FMT[fmt], Wd, xd, y, N, K))
        outs.append(y)
    lq.lq_gemv_batch(descs, ws=gu.gemv_ws())
    torch.cuda.synchronize()
    for (fmt, N, K, w, s, x), y in zip(cases, outs):
        gu.check_guard(y, N)
        yr, S = oracle.gemv(ORACLE_FMT[fmt], w, s, x, N, K)
        assert gu.ratio(y[:N].cpu().numpy(), yr, S, gu.GEMV_REL, gu.GEMV_ABS) <= 1.0, (fmt, N, K)


def test_graph_replays_match_eager(oracle):
    """GEMV launches that split K (per-device counters and partials), a
    grouped launch and a split-K GEMM (workspace + ordered reduction),
    captured in one graph and replayed several times with eager work of the
    same kernels in between: every replay equals the eager result bit for
    bit, and the eager result passes the oracle."""
    say("graph replays")
    gemv_cases = [("q8_0", 96, 4096, np.float32), ("i8b64", 300, 2048, np.float16), ("q4_0", 64, 896, np.float32)]
    descs, ref_data = [], []
    for i, (fmt, N, K, xdt) in enumerate(gemv_cases):
        w, s = make(fmt, 3100 + i, N, K)
        x = lqgen.activations(3200 + i, K, xdt)
        descs.append((gu.FMT[fmt], gu.upload(fmt, w, s, N, K), to_device(x), torch.zeros(N, device="cuda"), N, K))
        ref_data.append((fmt, w, s, x, N, K))
    M, Ng, Kg = 96, 200, 1024
    wg, _ = make("q4_0", 3300, Ng, Kg)
    Wg = gu.upload("q4_0", wg, None, Ng, Kg)
    Xg = to_device(lqgen.activations(3301, M * Kg, np.float16).reshape(M, Kg))
    Yg = torch.zeros(M * Ng, device="cuda")
    wsb = lq.lq_gemm_workspace_bytes(lq.LQ_Q4_0, M, Ng, Kg)
    assert wsb > 0, "shape meant to split K"
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")

    def run():
        lq.lq_gemv_batch([descs[0]], ws=gu.gemv_ws())
        lq.lq_gemv_batch(descs[1:], ws=gu.gemv_ws())
        lq.lq_gemm(lq.LQ_Q4_0, Wg, Xg, Yg, M, Ng, Kg, ws=ws, ws_bytes=wsb)

    outs = [d[3] for d in descs] + [Yg]
    run()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    for (fmt, w, s, x, N, K), y in zip(ref_data, eager):
        yr, S = oracle.gemv(ORACLE_FMT[fmt], w, s, x, N, K)
        assert gu.ratio(y.cpu().numpy(), yr, S, gu.GEMV_REL, gu.GEMV_ABS) <= 1.0, fmt
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
        run()                       # eager work of the same kernels between replays
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"eager run after replay {rep} differs"


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0", "i8b64", "i8b32"])
def test_gemv_invariants(oracle, fmt):
    N, K = 96, 2048 if fmt != "q4_0" else 896
    say("gemv invariants", fmt, N, K)
    w, s = make(fmt, 31337, N, K)
    x = lqgen.activations(7, K, np.float32)
    Wd = gu.upload(fmt, w, s, N, K)
    y1 = gu.gemv(fmt, Wd, x, N, K)
    y2 = gu.gemv(fmt, Wd, x, N, K)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), "not deterministic"
    # every scale doubled -> y doubles bit for bit
    if fmt in gu.PLANAR:
        w2, s2 = w, s * np.float32(2)
    else:
        bb = 18 if fmt == "q4_0" else 34
        blk = w.reshape(-1, bb).copy()
        d = blk[:, 0:2].copy().view(np.float16) * np.float16(2)
        blk[:, 0:2] = d.view(np.uint8).reshape(-1, 2)
        w2, s2 = blk.reshape(-1), None
    y3 = gu.gemv(fmt, gu.upload(fmt, w2, s2, N, K), x, N, K)
    assert np.array_equal(y3, 2 * y1)
    # one-hot x -> column of the unpacked weights, bit for bit
    out32 = torch.empty(N * K, dtype=torch.float32, device="cuda")
    lq.lq_dequant_f32(gu.FMT[fmt], Wd, out32, N, K)
    torch.cuda.synchronize()
    full = out32.cpu().numpy().reshape(N, K)
    for k in (0, 1, 15, 16, 31, 32, 63, K - 1):
        e = np.zeros(K, np.float32)
        e[k] = 1.0
        yk = gu.gemv(fmt, Wd, e, N, K)
        assert np.array_equal(yk.view(np.uint32), full[:, k].view(np.uint32)), k


def test_gemv_zero_codes():
    """Q4_0 codes all 8 (and Q8_0 codes all 0) give exactly zero."""
    N, K = 64, 896
    for fmt, byte in (("q4_0", 0x88), ("q8_0", 0x00)):
        say("gemv zero codes", fmt)
        w, _ = make(fmt, 5, N, K)
        bb = 18 if fmt == "q4_0" else 34
        blk = w.reshape(-1, bb).copy()
        blk[:, 2:] = byte
        y = gu.gemv(fmt, gu.upload(fmt, blk.reshape(-1), None, N, K),
                    lqgen.activations(3, K, np.float32), N, K)
        assert np.all(y == 0)


# ------------------------------------------------ workloads at full size ----

def _run_workload_rows(oracle, wl, sample=None, batch=True):
    mats = [(m, *m.generate()) for m in wl.mats]
    xs = {k: wl.x(k) for k in wl.xs}
    descs, outs, devs = [], [], []
    for m, w, s in mats:
        Wd = gu.upload(m.fmt, w, s, m.N, m.K)
        xd = to_device(xs[m.xkey])
        y = gu.guarded(m.N)
        devs.append((Wd, xd))
        descs.append((gu.FMT[m.fmt], Wd, xd, y, m.N, m.K))
        outs.append(y)
    if batch:
        lq.lq_gemv_batch(descs, ws=gu.gemv_ws())
    else:
        for d in descs:
            lq.lq_gemv(d[0], d[1], d[2], d[3], d[4], d[5], ws=gu.gemv_ws())
    torch.cuda.synchronize()
    worst = 0.0
    for (m, w, s), y in zip(mats, outs):
        gu.check_guard(y, m.N)
        yy = y[:m.N].cpu().numpy()
        if sample and m.N > sample:
            rng = np.random.default_rng(m.seed)
            rows = np.unique(np.concatenate([[0, 1, m.N - 2, m.N - 1], rng.integers(0, m.N, sample)]))
            yr, S = oracle.gemv(ORACLE_FMT[m.fmt], w, s, xs[m.xkey], m.N, m.K, rows=rows)
            r = gu.ratio(yy[rows], yr, S, gu.GEMV_REL, gu.GEMV_ABS)
        else:
            yr, S = oracle.gemv(ORACLE_FMT[m.fmt], w, s, xs[m.xkey], m.N, m.K)
            r = gu.ratio(yy, yr, S, gu.GEMV_REL, gu.GEMV_ABS)
        assert r <= 1.0, (wl.name, m.name, r)
        worst = max(worst, r)
    return worst


@pytest.mark.slow
def test_workload_q4_0_2560x960(oracle):
    say("workload q4_0 2560x960")
    _run_workload_rows(oracle, lqgen.q4_0_ffn_2560x960(), batch=False)


@pytest.mark.slow
def test_workload_q8_0_layer(oracle):
    say("workload q8_0 decoder layer (grouped launch)")
    _run_workload_rows(oracle, lqgen.q8_0_layer_2048(0), batch=True)


@pytest.mark.slow
def test_workload_q4_0_lm_head(oracle):
    """Every one of the 151,936 LM-head rows (and both FFN matrices)."""
    say("workload q4_0 LM head 151936x896 + FFN, every row")
    _run_workload_rows(oracle, lqgen.q4_0_lmhead_151936x896(), batch=False)


@pytest.mark.slow
def test_workload_i8b64_layers(oracle):
    """The first and last TinyLlama layers, every row, grouped as bench.py
    groups the whole set."""
    for layer in (0, 21):
        say("workload i8b64 TinyLlama layer", layer, "every row")
        _run_workload_rows(oracle, lqgen.i8b64_tinyllama_layer(layer), batch=True)


# ---------------------------------------------------------------- GEMM ----

# Covers row, column and K tails, odd block counts, and K split across
# workgroups (2 or 4 slices, uneven last slice).
GEMM_SHAPES = [(16, 64, 64), (5, 33, 96), (130, 129, 160), (1, 128, 64), (200, 300, 2048),
               (512, 256, 1024), (64, 2048, 1376), (96, 200, 1120), (300, 130, 1056),
               (257, 385, 512)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_parity(oracle, M, N, K):
    say("gemm", M, N, K)
    w, _ = make("q4_0", 77 + N, N, K)
    X = lqgen.activations(55 + M, M * K, np.float16).reshape(M, K)
    Wd = gu.upload("q4_0", w, None, N, K)
    Y = gu.gemm(Wd, X, M, N, K)
    Yr, S = oracle.gemm(0, w, None, X, M, N, K)
    assert gu.ratio(Y, Yr, S, gu.GEMM_REL, gu.GEMM_ABS) <= 1.0
    # against the fp16 tile contract the fp32-accumulation error is all that is left
    Yt, St = oracle.gemm(0, w, None, X, M, N, K, round_w_f16=True)
    assert gu.ratio(Y, Yt, St, 1e-4, 1e-6) <= 1.0


# Q8_0 and int8 block-64 prefill: row, column and K tails, K split across
# workgroups, several token blocks.
GEMM_INT8_SHAPES = [(16, 64, 64), (5, 33, 128), (130, 129, 256), (1, 128, 64), (200, 300, 2048),
                    (512, 256, 1024), (64, 2048, 1408), (96, 200, 1152), (257, 385, 512)]


@pytest.mark.parametrize("fmt", ["q8_0", "i8b64", "i8b32"])
@pytest.mark.parametrize("M,N,K", GEMM_INT8_SHAPES)
def test_gemm_int8_formats(oracle, fmt, M, N, K):
    """Against the exact product at the GEMM bar, and tightly against the
    format's tile contract: Q8_0 multiplies RN_fp16(c d) (the fp16 tile, as
    lq_dequant_f16), int8 block-64 keeps the codes exact and applies the fp32
    scale to each block sum, so only fp32 accumulation error remains."""
    say("gemm", fmt, M, N, K)
    w, s = make(fmt, 91 + N + K, N, K)
    X = lqgen.activations(57 + M, M * K, np.float16).reshape(M, K)
    Wd = gu.upload(fmt, w, s, N, K)
    Y = gu.gemm(Wd, X, M, N, K, fmt)
    Yr, S = oracle.gemm(ORACLE_FMT[fmt], w, s, X, M, N, K)
    assert gu.ratio(Y, Yr, S, gu.GEMM_REL, gu.GEMM_ABS) <= 1.0
    Yt, St = oracle.gemm(ORACLE_FMT[fmt], w, s, X, M, N, K, round_w_f16=(fmt == "q8_0"))
    assert gu.ratio(Y, Yt, St, 1e-4, 1e-6) <= 1.0


@pytest.mark.parametrize("fmt", ["q8_0", "i8b64", "i8b32"])
def test_gemm_int8_one_hot_rows(fmt):
    """X[m] = e_{k_m}: Q8_0 gives Y[m, :] = RN_fp16 of weight column k_m and
    int8 block-64 gives RN_fp32 of it (lq_dequant_f16 / lq_dequant_f32), bit
    for bit."""
    M, N, K = 72, 160, 384
    say("gemm one-hot", fmt, M, N, K)
    w, s = make(fmt, 6, N, K)
    Wd = gu.upload(fmt, w, s, N, K)
    ks = [(11 * m + 5) % K for m in range(M)]
    X = np.zeros((M, K), np.float16)
    for m, k in enumerate(ks):
        X[m, k] = 1
    Y = gu.gemm(Wd, X, M, N, K, fmt)
    if fmt == "q8_0":
        out = torch.empty(N * K, dtype=torch.uint16, device="cuda")
        lq.lq_dequant_f16(gu.FMT[fmt], Wd, out, N, K)
        torch.cuda.synchronize()
        ref = out.cpu().numpy().reshape(N, K).view(np.float16).astype(np.float32)
    else:
        out = torch.empty(N * K, dtype=torch.float32, device="cuda")
        lq.lq_dequant_f32(gu.FMT[fmt], Wd, out, N, K)
        torch.cuda.synchronize()
        ref = out.cpu().numpy().reshape(N, K)
    for m, k in enumerate(ks):
        assert np.array_equal(Y[m].view(np.uint32), ref[:, k].view(np.uint32)), m


def test_gemm_one_hot_rows_pin_tile():
    """X[m] = e_{k_m} gives Y[m, :] = RN_fp16 of weight column k_m, bit for bit."""
    M, N, K = 40, 160, 320
    say("gemm one-hot", M, N, K)
    w, _ = make("q4_0", 4, N, K)
    Wd = gu.upload("q4_0", w, None, N, K)
    ks = [(7 * m + 3) % K for m in range(M)]
    X = np.zeros((M, K), np.float16)
    for m, k in enumerate(ks):
        X[m, k] = 1
    Y = gu.gemm(Wd, X, M, N, K)
    out16 = torch.empty(N * K, dtype=torch.uint16, device="cuda")
    lq.lq_dequant_f16(lq.LQ_Q4_0, Wd, out16, N, K)
    torch.cuda.synchronize()
    W16 = out16.cpu().numpy().reshape(N, K).view(np.float16).astype(np.float32)
    for m, k in enumerate(ks):
        assert np.array_equal(Y[m].view(np.uint32), W16[:, k].view(np.uint32)), m


def test_gemm_rows_match_gemv(oracle):
    M, N, K = 48, 200, 2048
    say("gemm rows vs gemv", M, N, K)
    w, _ = make("q4_0", 8, N, K)
    Wd = gu.upload("q4_0", w, None, N, K)
    X = lqgen.activations(9, M * K, np.float16).reshape(M, K)
    Y = gu.gemm(Wd, X, M, N, K)
    for m in (0, 17, 47):
        y = gu.gemv("q4_0", Wd, X[m], N, K)
        _, S = oracle.gemv(0, w, None, X[m], N, K)
        assert np.all(np.abs(Y[m].astype(np.float64) - y) <= gu.GEMM_REL * S + gu.GEMM_ABS), m


def test_matmul_routes_by_token_count():
    N, K = 96, 256
    say("matmul routing")
    w, _ = make("q4_0", 12, N, K)
    Wd = gu.upload("q4_0", w, None, N, K)
    x = lqgen.activations(13, K, np.float16)
    y1 = gu.gemv("q4_0", Wd, x, N, K)
    Y = gu.guarded(N)
    lq.lq_matmul(lq.LQ_Q4_0, Wd, to_device(x), Y, 1, N, K, ws=gu.gemv_ws())
    torch.cuda.synchronize()
    assert np.array_equal(Y[:N].cpu().numpy(), y1)


def _prefill_ffn_all_outputs(oracle, fmt, fid, mats, X, M):
    """gate and up through one lq_gemm_batch launch, down through lq_gemm
    (K split across workgroups, workspace and ordered reduction), as bench.py
    times them; every output against the oracle at the GEMM bar."""
    byname = {name: (w, s, N, K) for name, w, s, N, K in mats}
    Wd = {name: gu.upload(fmt, w, s, N, K) for name, (w, s, N, K) in byname.items()}
    gate, up, down = byname["gate"], byname["up"], byname["down"]
    Xd = to_device(X["in"])
    Yg, Yu = gu.guarded(M * gate[2]), gu.guarded(M * up[2])
    say("gemm workload", fmt, "gate+up (one launch)", M, gate[2], gate[3])
    lq.lq_gemm_batch(fid, Xd, M, gate[3], [(Wd["gate"], Yg, gate[2]), (Wd["up"], Yu, up[2])])
    say("gemm workload", fmt, "down", M, down[2], down[3])
    wsb = lq.lq_gemm_workspace_bytes(fid, M, down[2], down[3])
    assert wsb > 0, "down is meant to split K"
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    Yd = gu.guarded(M * down[2])
    lq.lq_gemm(fid, Wd["down"], to_device(X["down"]), Yd, M, down[2], down[3], ws=ws)
    torch.cuda.synchronize()
    for name, Y, xk in (("gate", Yg, "in"), ("up", Yu, "in"), ("down", Yd, "down")):
        w, s, N, K = byname[name]
        gu.check_guard(Y, M * N)
        Yr, S = oracle.gemm(ORACLE_FMT[fmt], w, s, X[xk], M, N, K)
        r = gu.ratio(Y[:M * N].cpu().numpy().reshape(M, N), Yr, S, gu.GEMM_REL, gu.GEMM_ABS)
        assert r <= 1.0, (fmt, name, r)


@pytest.mark.slow
@pytest.mark.parametrize("fmt", ["q8_0", "i8b64", "i8b32"])
def test_workload_int8_prefill(oracle, fmt):
    """The prefill FFN shapes (2048 / 11008, M = 512) with int8 weights,
    every output against the exact product at the GEMM bar."""
    M = 512
    mats = []
    for name, N, K in (("gate", 11008, 2048), ("up", 11008, 2048), ("down", 2048, 11008)):
        w, s = make(fmt, 4400 + N + (1 if name == "up" else 0), N, K)
        mats.append((name, w, s, N, K))
    X = {"in": lqgen.activations(4500 + 2048, M * 2048, np.float16).reshape(M, 2048),
         "down": lqgen.activations(4500 + 11008, M * 11008, np.float16).reshape(M, 11008)}
    _prefill_ffn_all_outputs(oracle, fmt, gu.FMT[fmt], mats, X, M)


@pytest.mark.slow
def test_workload_q4_0_prefill_ffn(oracle):
    """The Q4_0 prefill FFN (2048 / 11008, M = 512) in bench.py's launches,
    every one of its 512 x (11008 + 11008 + 2048) outputs."""
    wl = lqgen.q4_0_prefill_ffn_2048x11008(512)
    mats = [(m.name, m.generate()[0], None, m.N, m.K) for m in wl.mats]
    keys = {m.name: m.xkey for m in wl.mats}
    X = {"in": wl.x(keys["gate"]), "down": wl.x(keys["down"])}
    assert keys["gate"] == keys["up"]
    _prefill_ffn_all_outputs(oracle, "q4_0", lq.LQ_Q4_0, mats, X, wl.M)
