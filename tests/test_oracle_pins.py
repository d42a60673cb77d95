"""Pins of the CPU oracle to facts outside itself (no GPU needed).

What pins what:
  * fp16 codec: all 65,536 bit patterns against numpy's own binary16 decoder,
    and the encoder against numpy's round-to-nearest-even cast from double
    (independent implementations of IEEE 754 binary16).
  * Block layouts: hand-built blocks H1-H5 (tests/golden/blocks.json) whose
    values were worked out by hand from the GGUF Q4_0 / Q8_0 definitions
    ("lean" page, model table: GGUF Q4_0 and Q8_0 files; "oxinfer" page,
    "How it works", quant.rs: two nibbles per byte, f16 scale).
  * int8 block-64 ("wgpu-llm" page, "INT8 mode", block size 64): exact products
    checked against numpy's IEEE fp32 multiply (single rounding).
  * GEMV / GEMM: brute force with exact rational arithmetic on tiny matrices,
    closed forms (all codes 8 -> 0, one-hot x -> a column, ones -> row sums),
    cross-format identities and scale linearity.
Each pin is a function of an oracle build, so test_oracle_mutants.py can run the
same pins against copies of the oracle with a planted mistake.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

Q4_0, Q8_0, I8B64, I8B32 = 0, 1, 2, 3
GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "blocks.json")))


def _f16(v):
    with np.errstate(over="ignore"):
        return np.array([v], np.float64).astype(np.float16).view(np.uint16)[0]


# ---------------------------------------------------------------- fp16 codec

def pin_half_decode(o):
    ref = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float64)
    got = np.array([o.half_to_double(h) for h in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint64), ref[~nan].view(np.uint64))  # sign of 0 too


def pin_half_encode(o):
    rng = np.random.default_rng(1234)
    vals = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-9, 6, 3000))
    # exact halfway cases between adjacent fp16 values, in every binade
    h = np.arange(0, 0x7BFF, 37, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    vals += list((lo + hi) / 2) + list(-(lo + hi) / 2)
    vals += [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9, np.inf, -np.inf,
             2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 2.0 ** -14,
             2.0 ** -14 - 2.0 ** -25]
    for v in vals:
        want = int(_f16(v))
        got = o.double_to_half(v)
        assert got == want, (v, hex(got), hex(want))
    assert o.double_to_half(np.nan) & 0x7C00 == 0x7C00 and o.double_to_half(np.nan) & 0x3FF


# ----------------------------------------------------------- hand-built blocks

def _fmt(name):
    return {"q4_0": Q4_0, "q8_0": Q8_0}[name]


def pin_golden_blocks(o):
    for blk in GOLD["blocks"]:
        raw = np.frombuffer(bytes.fromhex(blk["hex"]), np.uint8).copy()
        fmt = _fmt(blk["fmt"])
        assert len(raw) == o.gguf_block_bytes(fmt)
        want = np.array([float(s) for s in blk["expected"]])
        got = o.dequant(fmt, raw, None, 1, 32)[0]
        assert np.array_equal(got.view(np.uint64), want.view(np.uint64)), blk["id"]
        got32 = o.dequant_f32(fmt, raw, None, 1, 32)[0]
        assert np.array_equal(got32.view(np.uint32), want.astype(np.float32).view(np.uint32)), blk["id"]
        f16 = blk.get("f16", blk["expected"])
        want16 = np.array([float(s) for s in f16]).astype(np.float16).view(np.uint16)
        assert np.array_equal(o.dequant_f16(fmt, raw, None, 1, 32)[0], want16), blk["id"]
        # GEMV with x = ones gives the block sum exactly
        y, S = o.gemv(fmt, raw, None, np.ones(32, np.float32), 1, 32)
        assert y[0] == float(blk["sum"]), blk["id"]
        assert S[0] == np.abs(want).sum(), blk["id"]


def pin_i8b64_single_rounding(o):
    s = np.float32(0.003)
    codes = np.full(64, 127, np.int8)
    scales = np.array([s], np.float32)
    exact = o.dequant(I8B64, codes, scales, 1, 64)[0]
    assert np.all(exact == 127.0 * float(s))            # exact product in double
    f32 = o.dequant_f32(I8B64, codes, scales, 1, 64)[0]
    want = np.float32(127) * s                          # one IEEE fp32 multiply
    assert np.all(f32.view(np.uint32) == np.array([want]).view(np.uint32)[0])
    assert float(want) != 127.0 * float(s)              # the rounding is visible
    # code -128 decodes as -128 and the second half-block uses the same scale
    codes2 = np.arange(-64, 64, dtype=np.int64).astype(np.int8)
    sc2 = np.array([0.5, 0.25], np.float32)
    d = o.dequant(I8B64, codes2, sc2, 1, 128)[0]
    assert d[0] == -32.0 and d[63] == -0.5 and d[64] == 0.0 and d[127] == 63 * 0.25


def _half_of_exact(c, s):
    """numpy's direct double -> binary16 cast (round to nearest even, one
    rounding) of the exact product c * s."""
    with np.errstate(over="ignore"):
        return (np.asarray(c, np.float64) * np.asarray(s, np.float32).astype(np.float64)).astype(np.float16).view(np.uint16)


def _double_rounding_cases():
    """(code, fp32 scale) pairs whose exact product lies just off an fp16
    halfway point, inside half an fp32 ulp of it: rounding the product to
    fp32 first lands on the halfway point and then ties to even, which is
    not RN_fp16 of the exact product.  Found by search, checked here."""
    rng = np.random.default_rng(2024)
    cases = []
    for h in rng.integers(0x0001, 0x7BFE, 300).astype(np.uint16):
        lo, hi = np.array([h, h + 1], np.uint16).view(np.float16).astype(np.float64)
        t = (lo + hi) / 2
        for c in (3, 5, 7, 11, 13, 127, -3, -9, -117):
            s0 = np.float32(t / c)
            for s in (np.nextafter(s0, np.float32(-np.inf)), s0, np.nextafter(s0, np.float32(np.inf))):
                p = float(c) * float(s)
                via32 = np.array([np.float32(p)], np.float32).astype(np.float16).view(np.uint16)[0]
                if _half_of_exact(c, s) != via32:
                    cases.append((c, s))
    assert len(cases) > 100
    return cases


def pin_int8_f16_single_rounding(o):
    """dequant_f16 of the fp32-scale formats is RN_fp16 of the exact product
    c * s, rounded once from the exact value (numpy's double -> half cast):
    random codes and scales in the generated ranges and above, products
    that a rounding through fp32 would move (double rounding), exact ties,
    fp16 subnormals and overflow to inf."""
    rng = np.random.default_rng(77)
    pairs = _double_rounding_cases()
    # exact halfway points between fp16 neighbours, as c * s with c = +-1, +-2
    h = rng.integers(0x0001, 0x7BFE, 200).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    for c, m in ((1, (lo + hi) / 2), (-2, (lo + hi) / 4)):
        pairs += [(c, np.float32(v)) for v in m if float(np.float32(v)) == v]
    # subnormal results (and their halfway points), the largest finite value
    # and the overflow boundary 65520
    pairs += [(1, np.float32(2.0 ** -25)), (3, np.float32(2.0 ** -25)), (5, np.float32(2.0 ** -26)),
              (1, np.float32(2.0 ** -24 * 1.5)), (-1, np.float32(2.0 ** -24 * 2.5)), (7, np.float32(1e-9)),
              (127, np.float32(65504.0 / 127)), (1, np.float32(65504.0)), (1, np.float32(65519.0)),
              (2, np.float32(32760.0)), (-2, np.float32(32760.0)), (127, np.float32(600.0)),
              (1, np.float32(65520.0)), (0, np.float32(3.0)), (-128, np.float32(0.5))]
    for fmt, E in ((I8B64, 64), (I8B32, 32)):
        # one code and one scale per block: the tested pair sits at element 0
        # of its block, the rest of the block are random codes
        nb = len(pairs)
        K = E * 4
        N = (nb + 3) // 4
        codes = rng.integers(-127, 128, N * K).astype(np.int8)
        scales = (np.abs(rng.standard_normal(N * 4)) * rng.choice([0.003, 0.5, 20.0], N * 4)).astype(np.float32)
        for i, (c, s) in enumerate(pairs):
            codes[i * E] = c
            scales[i] = s
        got = o.dequant_f16(fmt, codes, scales, N, K).reshape(-1)
        want = _half_of_exact(codes.astype(np.float64), np.repeat(scales, E))
        assert np.array_equal(got, want), fmt


# ----------------------------------------------------------------- brute force

def _q4_block_bytes(codes32, dbits):
    """Pack one Q4_0 block by the definition: byte j = c[j] | c[j+16] << 4."""
    b = [dbits & 0xFF, dbits >> 8] + [int(codes32[j]) | (int(codes32[j + 16]) << 4) for j in range(16)]
    return b


def _q8_block_bytes(codes32, dbits):
    return [dbits & 0xFF, dbits >> 8] + [int(c) & 0xFF for c in codes32]


def pin_bruteforce(o):
    rng = np.random.default_rng(7)
    for fmt in (Q4_0, Q8_0):
        for N in (1, 2, 3, 4):
            for K in (32, 64, 96, 128):
                nb = K // 32
                if fmt == Q4_0:
                    codes = rng.integers(0, 16, (N, K))
                    vals = codes - 8
                else:
                    codes = rng.integers(-128, 128, (N, K))
                    vals = codes
                exps = rng.integers(-10, 6, (N, nb))
                raw = []
                for n in range(N):
                    for b in range(nb):
                        dbits = int(_f16(2.0 ** int(exps[n, b])))
                        c = codes[n, b * 32:(b + 1) * 32]
                        raw += _q4_block_bytes(c, dbits) if fmt == Q4_0 else _q8_block_bytes(c, dbits)
                raw = np.array(raw, np.uint8)
                x = rng.integers(-9, 10, K).astype(np.float32)
                y, S = o.gemv(fmt, raw, None, x, N, K)
                for n in range(N):
                    yy = sum(Fraction(int(vals[n, k])) * Fraction(2) ** int(exps[n, k // 32]) * int(x[k])
                             for k in range(K))
                    ss = sum(abs(Fraction(int(vals[n, k])) * Fraction(2) ** int(exps[n, k // 32]) * int(x[k]))
                             for k in range(K))
                    assert Fraction(y[n]) == yy and Fraction(S[n]) == ss, (fmt, N, K, n)
    # int8 block-64 with power-of-two fp32 scales
    for N in (1, 3):
        for K in (64, 128, 192):
            codes = rng.integers(-128, 128, (N, K)).astype(np.int8)
            exps = rng.integers(-20, 4, (N, K // 64))
            sc = (2.0 ** exps).astype(np.float32)
            x = rng.integers(-9, 10, K).astype(np.float16)
            y, _ = o.gemv(I8B64, codes, sc, x, N, K)
            for n in range(N):
                yy = sum(Fraction(int(codes[n, k])) * Fraction(2) ** int(exps[n, k // 64]) * int(x[k])
                         for k in range(K))
                assert Fraction(y[n]) == yy


# ------------------------------------------------------ closed forms, identities

def _rand_q4(rng, N, K):
    nb = N * K // 32
    blk = np.empty((nb, 18), np.uint8)
    blk[:, :2] = (np.abs(rng.standard_normal(nb)) * 0.02).astype(np.float16).view(np.uint8).reshape(nb, 2)
    blk[:, 2:] = rng.integers(0, 256, (nb, 16))
    return blk.reshape(-1)


def pin_closed_forms(o):
    rng = np.random.default_rng(11)
    N, K = 5, 96
    # every code 8 -> w = 0 -> y = 0 exactly for any x
    w8 = _rand_q4(rng, N, K).reshape(-1, 18)
    w8[:, 2:] = 0x88
    x = rng.standard_normal(K).astype(np.float32)
    y, S = o.gemv(Q4_0, w8.reshape(-1), None, x, N, K)
    assert np.all(y == 0) and np.all(S == 0)
    # one-hot x = e_k -> y = column k of the decoded matrix, bit for bit
    w = _rand_q4(rng, N, K)
    full = o.dequant(Q4_0, w, None, N, K)
    for k in (0, 1, 15, 16, 17, 31, 32, 63, 95):
        e = np.zeros(K, np.float32)
        e[k] = 1.0
        y, _ = o.gemv(Q4_0, w, None, e, N, K)
        assert np.array_equal(y, full[:, k]), k
    # d = 1, x = ones -> integer row sums of (q - 8), from the nibbles themselves
    w1 = w.reshape(-1, 18).copy()
    w1[:, 0], w1[:, 1] = 0x00, 0x3C
    y, _ = o.gemv(Q4_0, w1.reshape(-1), None, np.ones(K, np.float32), N, K)
    nib = w1[:, 2:].reshape(N, -1, 16)
    rows = ((nib & 15).astype(int) - 8).sum(axis=(1, 2)) + ((nib >> 4).astype(int) - 8).sum(axis=(1, 2))
    assert np.array_equal(y, rows.astype(np.float64))


def pin_cross_format(o):
    rng = np.random.default_rng(5)
    N, K = 4, 128
    nb = K // 32
    codes = rng.integers(0, 16, (N, K))
    dbits = (np.abs(rng.standard_normal(N * nb)) * 0.05).astype(np.float16).view(np.uint16)
    q4, q8 = [], []
    for n in range(N):
        for b in range(nb):
            c = codes[n, b * 32:(b + 1) * 32]
            q4 += _q4_block_bytes(c, int(dbits[n * nb + b]))
            q8 += _q8_block_bytes(c - 8, int(dbits[n * nb + b]))
    q4, q8 = np.array(q4, np.uint8), np.array(q8, np.uint8)
    assert np.array_equal(o.dequant(Q4_0, q4, None, N, K), o.dequant(Q8_0, q8, None, N, K))
    x = rng.standard_normal(K).astype(np.float32)
    assert np.array_equal(o.gemv(Q4_0, q4, None, x, N, K)[0], o.gemv(Q8_0, q8, None, x, N, K)[0])
    # I8B64 block with an fp16-representable scale == two Q8_0 blocks with that scale
    c8 = rng.integers(-127, 128, (N, K)).astype(np.int8)
    s64 = np.abs(rng.standard_normal(N * K // 64) * 0.01).astype(np.float16)
    q8b = []
    for n in range(N):
        for b in range(nb):
            q8b += _q8_block_bytes(c8[n, b * 32:(b + 1) * 32], int(s64[(n * K + b * 32) // 64].view(np.uint16)))
    q8b = np.array(q8b, np.uint8)
    assert np.array_equal(o.dequant(I8B64, c8.reshape(-1), s64.astype(np.float32), N, K),
                          o.dequant(Q8_0, q8b, None, N, K))


def pin_i8b32_against_other_formats(o):
    """The "oxinfer" page's Q8 (int8 codes, one fp32 scale per 32) pinned to
    the independently pinned formats: with each 64-block's scale repeated
    for both of its halves it is I8B64 exactly; with fp16-representable
    scales it is Q8_0 exactly (dequant and GEMV); its quantizer on a
    32-block h equals the I8B64 quantizer on the 64-block [h, h]."""
    rng = np.random.default_rng(23)
    N, K = 5, 128
    c = rng.integers(-127, 128, (N, K)).astype(np.int8)
    s64 = (np.abs(rng.standard_normal(N * K // 64)) * 0.01).astype(np.float32)
    s32 = np.repeat(s64, 2)
    assert np.array_equal(o.dequant(I8B32, c.reshape(-1), s32, N, K), o.dequant(I8B64, c.reshape(-1), s64, N, K))
    s16 = (np.abs(rng.standard_normal(N * K // 32)) * 0.01).astype(np.float16)
    q8 = []
    for n in range(N):
        for b in range(K // 32):
            q8 += _q8_block_bytes(c[n, b * 32:(b + 1) * 32], int(s16[n * (K // 32) + b].view(np.uint16)))
    q8 = np.array(q8, np.uint8)
    assert np.array_equal(o.dequant(I8B32, c.reshape(-1), s16.astype(np.float32), N, K),
                          o.dequant(Q8_0, q8, None, N, K))
    x = rng.standard_normal(K).astype(np.float32)
    assert np.array_equal(o.gemv(I8B32, c.reshape(-1), s16.astype(np.float32), x, N, K)[0],
                          o.gemv(Q8_0, q8, None, x, N, K)[0])
    w = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    q32, sc32 = o.quantize(I8B32, w, N, K)
    dup = np.concatenate([np.repeat(w.reshape(N, K // 32, 1, 32), 2, axis=2)], axis=0).reshape(N, 2 * K)
    q64, sc64 = o.quantize(I8B64, dup, N, 2 * K)
    q64 = q64.reshape(N, K // 32, 2, 32)
    assert np.array_equal(q32.reshape(N, K // 32, 32), q64[:, :, 0, :])
    assert np.array_equal(q64[:, :, 0, :], q64[:, :, 1, :])
    assert np.array_equal(sc32.view(np.uint32), sc64.view(np.uint32))


def pin_scale_linearity_and_gemm(o):
    rng = np.random.default_rng(9)
    N, K, M = 6, 64, 5
    w = _rand_q4(rng, N, K)
    x = rng.standard_normal(K).astype(np.float32)
    y, _ = o.gemv(Q4_0, w, None, x, N, K)
    w2 = w.reshape(-1, 18).copy()
    d = w2[:, :2].copy().view(np.uint16).view(np.float16).astype(np.float64) * 2
    w2[:, :2] = d.astype(np.float16).view(np.uint16).view(np.uint8).reshape(-1, 2)
    y2, _ = o.gemv(Q4_0, w2.reshape(-1), None, x, N, K)
    assert np.array_equal(y2, 2 * y)
    # GEMM: Y = X W^T; row m of Y equals the GEMV of X[m] (same sum order)
    X = rng.standard_normal((M, K)).astype(np.float16)
    Y, SY = o.gemm(Q4_0, w, None, X, M, N, K)
    for m in range(M):
        ym, sm = o.gemv(Q4_0, w, None, X[m], N, K)
        assert np.array_equal(Y[m], ym) and np.array_equal(SY[m], sm)
    # one-hot token rows X[m] = e_{k_m} -> Y[m, :] = column k_m of the weights;
    # with the fp16 tile contract, Y[m, :] = RN_fp16 of that column
    ks = [0, 16, 33, 63, 40]
    E = np.zeros((M, K), np.float16)
    for m, k in enumerate(ks):
        E[m, k] = 1
    full = o.dequant(Q4_0, w, None, N, K)
    Ye, _ = o.gemm(Q4_0, w, None, E, M, N, K)
    Yr, _ = o.gemm(Q4_0, w, None, E, M, N, K, round_w_f16=True)
    for m, k in enumerate(ks):
        assert np.array_equal(Ye[m], full[:, k])
        assert np.array_equal(Yr[m], full[:, k].astype(np.float16).astype(np.float64))
    # a row subset gives the same numbers as the full product
    Ys, _ = o.gemm(Q4_0, w, None, X, M, N, K, ms=[4, 1], ns=[5, 0, 2])
    assert np.array_equal(Ys, Y[[4, 1]][:, [5, 0, 2]])


def pin_roundtrip(o):
    rng = np.random.default_rng(3)
    N, K = 7, 160
    for fmt, lo, hi in ((Q4_0, 0, 16), (Q8_0, -128, 128)):
        codes = rng.integers(lo, hi, (N, K)).astype(np.int8)
        sb = rng.integers(0, 0x7C00, (N, K // 32)).astype(np.uint16)
        sb[0, 0] |= 0x8000
        aos = o.pack_gguf(fmt, codes, sb, N, K)
        assert len(aos) == N * (K // 32) * o.gguf_block_bytes(fmt)
        c2, s2 = o.unpack_gguf(fmt, aos, N, K)
        assert np.array_equal(c2, codes) and np.array_equal(s2, sb)
        # pack follows the byte layout fixed by the hand-built blocks
        if fmt == Q4_0:
            b0 = aos[:18]
            assert b0[0] == sb[0, 0] & 0xFF and b0[1] == sb[0, 0] >> 8
            assert all(int(b0[2 + j]) == (int(codes[0, j]) | (int(codes[0, j + 16]) << 4)) for j in range(16))


def pin_byte_accounting(o):
    # "Q8 cuts them by 1.8x and Q4 by 3.5x" vs bf16 ("oxinfer" page, Performance):
    # Q4_0 is 18 bytes per 32 weights; the page's Q8 keeps an f32 scale
    # (36 bytes per 32), while GGUF Q8_0 (fp16 scale) is 34 bytes per 32.
    assert o.block_elems(Q4_0) == 32 and o.gguf_block_bytes(Q4_0) == 18
    assert o.block_elems(Q8_0) == 32 and o.gguf_block_bytes(Q8_0) == 34
    assert o.block_elems(I8B64) == 64
    assert o.block_elems(I8B32) == 32 and o.gguf_block_bytes(I8B32) == 0
    assert round(2.0 / (18 / 32), 1) in (3.5, 3.6)
    assert round(2.0 / (36 / 32), 1) == 1.8


def pin_argument_checks(o):
    with pytest.raises(ValueError):
        o.dequant(Q4_0, np.zeros(18, np.uint8), None, 1, 33)    # K not a multiple of 32
    with pytest.raises(ValueError):
        o.dequant(I8B64, np.zeros(32, np.int8), np.zeros(1, np.float32), 1, 32)


ALL_PINS = [pin_half_decode, pin_half_encode, pin_golden_blocks, pin_i8b64_single_rounding,
            pin_bruteforce, pin_closed_forms, pin_cross_format, pin_scale_linearity_and_gemm,
            pin_roundtrip, pin_byte_accounting, pin_argument_checks, pin_i8b32_against_other_formats,
            pin_int8_f16_single_rounding]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(oracle, pin):
    pin(oracle)


def test_generator_splitmix64_published_values():
    """SplitMix64 seeded with 0: the first outputs of the published generator."""
    import lqgen
    z = lqgen.splitmix64(0, 3)
    assert [int(v) for v in z] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_generator_recipes_shapes():
    import lqgen
    w, s = lqgen.q4_0_ffn_2560x960().mats[0].generate()
    assert s is None and w.size == 2560 * 30 * 18
    c, sc = lqgen.i8b64_planes(1, 4, 128)
    assert c.dtype == np.int8 and c.size == 512 and sc.size == 8 and c.min() >= -127
    wl = lqgen.q8_0_layer_2048()
    assert wl.weight_bytes == 71303168
    assert lqgen.q4_0_lmhead_151936x896().mats[0].packed_bytes == 76575744
