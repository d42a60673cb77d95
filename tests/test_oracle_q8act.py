"""Pins of the oracle's activation-quantized integer-dot path (no GPU needed).

The "oxinfer" page ("How it works", quant.rs) quantizes activations for each
matmul and takes int8 dot products with the weight codes, four blocks at a
time, with multi-token variants; it gives no rounding rule.  The reading
pinned here: each 32-element block of a token row gets s = max|x| / 127 and
q = clamp(rint(x / s), +-127) in fp32 steps (the page's own Q8 rule), and the
product is Y[m,n] = sum_b ws(n,b) s[m,b] I(m,n,b) with I the exact integer
block dot product.

What pins what:
  * the quantizer: hand-derived blocks (plain values, exact ties to even, a
    zero block, a negative extreme, fp16 sources), idempotence on values that
    already are codes times a power-of-two scale, the |x - q s| <= s/2 bound;
  * the product: brute force with exact rationals on tiny matrices of every
    format, and agreement with the exact-activation GEMV oracle (already
    pinned) whenever the activations are exactly codes times scales.
Each pin is a function of an oracle build, so test_oracle_mutants.py runs
them against copies of the oracle with a planted mistake.
"""
from fractions import Fraction

import numpy as np
import pytest

import lqgen

Q4_0, Q8_0, I8B64, I8B32 = 0, 1, 2, 3


def pin_act_hand_block(o):
    # 3 is the largest magnitude: s = RN32(3 / 127); 0.5 / s = 21.17 -> 21,
    # -1 / s = -42.33 -> -42, 3 / s = 127, 0.25 / s = 10.58 -> 11
    x = np.array([[0.5, -1.0, 3.0, 0.25] * 8], np.float32)
    q, s, t = o.quantize_act(x, 1, 32)
    assert s[0, 0] == np.float32(3.0) / np.float32(127.0)
    assert list(q[0, :4]) == [21, -42, 127, 11] and np.array_equal(q[0], np.tile(q[0, :4], 8))
    assert t[0, 0] == 8 * (21 - 42 + 127 + 11)


def pin_act_ties_to_even(o):
    # max |x| = 127 makes s exactly 1, so x / s = x: halves round to even
    vals = [127.0, 2.5, 3.5, -2.5, -0.5, 0.5, 126.5, -126.5, 1.5, -1.5, 4.5, 0.0] + [0.0] * 20
    want = [127, 2, 4, -2, 0, 0, 126, -126, 2, -2, 4, 0] + [0] * 20
    x = np.array([vals], np.float32)
    q, s, t = o.quantize_act(x, 1, 32)
    assert s[0, 0] == 1.0
    assert list(q[0]) == want
    assert t[0, 0] == sum(want)


def pin_act_zero_and_negative_extreme(o):
    x = np.zeros((2, 64), np.float32)
    x[1, 32:] = np.linspace(-0.5, 0.9, 32)
    x[1, 40] = -7.0                      # the extreme is negative: it becomes -127
    q, s, t = o.quantize_act(x, 2, 64)
    assert np.all(q[0] == 0) and np.all(s[0] == 0) and np.all(t[0] == 0)
    assert np.all(q[1, :32] == 0) and s[1, 0] == 0
    assert s[1, 1] == np.float32(7.0) / np.float32(127.0)
    assert q[1, 40] == -127 and np.abs(q[1, 32:]).max() == 127


def pin_act_fp16_source(o):
    rng = np.random.default_rng(5)
    x16 = rng.standard_normal((3, 96)).astype(np.float16)
    a = o.quantize_act(x16, 3, 96)
    b = o.quantize_act(x16.astype(np.float32), 3, 96)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def pin_act_idempotent_and_bound(o):
    rng = np.random.default_rng(6)
    M, K = 4, 128
    c = rng.integers(-127, 128, (M, K)).astype(np.int64)
    c[:, ::32] = 127                                  # every block reaches the extreme code
    s0 = np.float32(2.0 ** -7)
    x = (c * float(s0)).astype(np.float32)            # exact: 8-bit code times a power of two
    q, s, _ = o.quantize_act(x, M, K)
    assert np.all(s == s0) and np.array_equal(q.astype(np.int64), c)
    # random activations: |x - q s| <= s / 2 (plus the fp32 division's rounding)
    xr = (rng.standard_normal((M, K)) * 3).astype(np.float32)
    q, s, t = o.quantize_act(xr, M, K)
    se = np.repeat(s, 32, axis=1).astype(np.float64)
    assert np.all(np.abs(xr - q * se) <= se / 2 * (1 + 2.0 ** -20))
    assert np.abs(q.astype(int)).max() <= 127
    assert np.all(np.abs(q.reshape(M, K // 32, 32)).max(axis=2) == 127)
    assert np.array_equal(t, q.reshape(M, K // 32, 32).astype(np.int32).sum(axis=2))


def _codes_and_scales(fmt, N, K, rng):
    """Random weights of a format as (bytes or codes, scales) plus the integer
    codes c[n, k] and exact scales ws[n, k] per element, built from the block
    definitions."""
    if fmt in (Q4_0, Q8_0):
        nb = K // 32
        d = (np.abs(rng.standard_normal(N * nb)) * 0.02).astype(np.float16)
        if fmt == Q4_0:
            qq = rng.integers(0, 16, (N, K))
            blk = np.zeros((N, nb, 18), np.uint8)
            blk[:, :, 0:2] = d.view(np.uint8).reshape(N, nb, 2)
            for j in range(16):
                blk[:, :, 2 + j] = qq.reshape(N, nb, 32)[:, :, j] | (qq.reshape(N, nb, 32)[:, :, j + 16] << 4)
            c = qq - 8
        else:
            c = rng.integers(-127, 128, (N, K))
            blk = np.zeros((N, nb, 34), np.uint8)
            blk[:, :, 0:2] = d.view(np.uint8).reshape(N, nb, 2)
            blk[:, :, 2:] = c.reshape(N, nb, 32).astype(np.int8).view(np.uint8)
        ws = np.repeat(d.reshape(N, nb), 32, axis=1)
        return blk.reshape(-1), None, c, ws
    E = 64 if fmt == I8B64 else 32
    c = rng.integers(-127, 128, (N, K))
    sc = (np.abs(rng.standard_normal(N * (K // E))) * 0.003).astype(np.float32)
    ws = np.repeat(sc.reshape(N, K // E), E, axis=1)
    return c.astype(np.int8).reshape(-1), sc, c, ws


def pin_q8act_bruteforce(o):
    rng = np.random.default_rng(7)
    M, N, K = 3, 5, 128
    for fmt in (Q4_0, Q8_0, I8B64, I8B32):
        w, sc, c, ws = _codes_and_scales(fmt, N, K, rng)
        x = rng.standard_normal((M, K)).astype(np.float32)
        q, s, _ = o.quantize_act(x, M, K)
        Y, S = o.gemv_q8act(fmt, w, sc, q, s, M, N, K)
        for m in range(M):
            for n in range(N):
                acc, aacc = Fraction(0), Fraction(0)
                for b in range(K // 32):
                    I = int(sum(int(c[n, k]) * int(q[m, k]) for k in range(32 * b, 32 * b + 32)))
                    t = Fraction(float(ws[n, 32 * b])) * Fraction(float(s[m, b])) * I
                    acc += t
                    aacc += abs(t)
                assert abs(Fraction(Y[m, n]) - acc) <= abs(aacc) * Fraction(1, 2 ** 50), (fmt, m, n)
                assert abs(Fraction(S[m, n]) - aacc) <= aacc * Fraction(1, 2 ** 50), (fmt, m, n)


def pin_q8act_matches_exact_gemv(o):
    # activations that are exactly codes x power-of-two scales quantize to
    # themselves, so the integer-dot product is the exact product W x
    rng = np.random.default_rng(8)
    M, K = 2, 256
    for fmt, N in ((Q4_0, 7), (Q8_0, 6), (I8B64, 5), (I8B32, 4)):
        wl = {Q4_0: lqgen.q4_0_aos, Q8_0: lqgen.q8_0_aos}
        if fmt in wl:
            w, sc = wl[fmt](40 + fmt, N, K), None
        else:
            w, sc = lqgen.i8_planes(40 + fmt, N, K, 64 if fmt == I8B64 else 32)
        cx = rng.integers(-127, 128, (M, K))
        cx[:, ::32] = -127
        x = (cx * 2.0 ** -6).astype(np.float32)
        q, s, _ = o.quantize_act(x, M, K)
        Y, _ = o.gemv_q8act(fmt, w, sc, q, s, M, N, K)
        for m in range(M):
            y, _ = o.gemv(fmt, w, sc, x[m], N, K)
            assert np.allclose(Y[m], y, rtol=1e-14, atol=1e-300), fmt


Q8ACT_PINS = [pin_act_hand_block, pin_act_ties_to_even, pin_act_zero_and_negative_extreme, pin_act_fp16_source,
              pin_act_idempotent_and_bound, pin_q8act_bruteforce, pin_q8act_matches_exact_gemv]


@pytest.mark.parametrize("pin", Q8ACT_PINS, ids=lambda f: f.__name__)
def test_q8act_pin(oracle, pin):
    pin(oracle)
