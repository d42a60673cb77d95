"""Pins of the oracle's load-time quantizer (lqref_quantize).

The pages give no rounding rule for load-time quantization, so the oracle
implements a stated reading (lqref.h): Q8_0 d = fp16(max|w| / 127), Q4_0
d = fp16(m / -8) with m the first element of largest magnitude, int8
block-64 s = max|w| / 127 in fp32, codes rint(w / d) (ties to even) clamped
to the format's range.  These tests pin it against facts that do not come
from retyping it: hand-derived blocks, exact idempotence on weights that are
already quantized, the rounding error bound, and agreement of the three
source types on values all of them hold exactly.
"""
import numpy as np
import pytest

import lqgen
from oracle import lqref

Q4, Q8, I8 = lqref.Q4_0, lqref.Q8_0, lqref.I8B64


def _codes_scales(o, fmt, out, scales, N, K):
    if fmt == I8:
        return out.reshape(N, K), scales.reshape(N, K // 64)
    c, s = o.unpack_gguf(fmt, out, N, K)
    return c, s


def pin_quant_hand_blocks(o):
    # Q8_0: max |w| = 127 -> d = 1 exactly; codes are w rounded to nearest
    # even: 2.5 -> 2, 3.5 -> 4, -2.5 -> -2, 126.6 -> 127, -0.5 -> -0 = 0.
    w = np.zeros((1, 32), np.float32)
    w[0, :8] = [-127.0, 2.5, 3.5, -2.5, 0.4999, 126.6, -0.5, 1.5]
    c, s = _codes_scales(o, Q8, *o.quantize(Q8, w, 1, 32), 1, 32)
    assert s[0, 0] == 0x3C00
    assert list(c[0, :8]) == [-127, 2, 4, -2, 0, 127, 0, 2]
    # Q4_0: -4 is the first element of largest magnitude (ties with +4), so
    # d = -4 / -8 = 0.5; 1.75 / 0.5 = 3.5 -> 4 -> code 12; -4 -> -8 -> code 0;
    # +4 -> +8 clamps to 7 -> code 15; 0.25 / 0.5 = 0.5 -> 0 -> code 8.
    w4 = np.zeros((1, 32), np.float32)
    w4[0, :4] = [1.75, -4.0, 4.0, 0.25]
    c4, s4 = _codes_scales(o, Q4, *o.quantize(Q4, w4, 1, 32), 1, 32)
    assert s4[0, 0] == 0x3800
    assert list(c4[0, :5]) == [12, 0, 15, 8, 8]
    # The sign of m decides: +4 first gives d = -0.5 and +4 -> code 0.
    w4[0, :4] = [1.75, 4.0, -4.0, 0.25]
    c4, s4 = _codes_scales(o, Q4, *o.quantize(Q4, w4, 1, 32), 1, 32)
    assert s4[0, 0] == 0xB800
    assert list(c4[0, :4]) == [4, 0, 15, 8]
    # int8 block-64: max |w| = 254 -> s = 2 exactly; 3 / 2 = 1.5 -> 2,
    # 5 / 2 = 2.5 -> 2, -7 / 2 = -3.5 -> -4.
    w8 = np.zeros((1, 64), np.float32)
    w8[0, :4] = [254.0, 3.0, 5.0, -7.0]
    c8, s8 = _codes_scales(o, I8, *o.quantize(I8, w8, 1, 64), 1, 64)
    assert s8[0, 0] == np.float32(2.0)
    assert list(c8[0, :4]) == [127, 2, 2, -4]


def pin_quant_zero_blocks(o):
    for fmt, K in ((Q8, 32), (Q4, 32), (I8, 64)):
        c, s = _codes_scales(o, fmt, *o.quantize(fmt, np.zeros((2, K), np.float32), 2, K), 2, K)
        assert np.all(c == (8 if fmt == Q4 else 0))
        assert np.all(np.asarray(s, np.float64) == 0) if fmt == I8 else np.all((s & 0x7FFF) == 0)


def pin_quant_idempotent(o):
    for fmt in (Q8, Q4, I8):
        _idempotent(o, fmt)


def _idempotent(o, fmt):
    """Weights that are already codes times a positive scale, with the
    extreme code present in every block (127 for Q8_0 / int8, 0 for Q4_0),
    quantize back to the same codes and scales exactly."""
    N, K = 7, 256
    rng = np.random.default_rng(5 + fmt)
    E = 64 if fmt == I8 else 32
    if fmt == Q4:
        codes = rng.integers(0, 16, (N, K)).astype(np.int8)
        codes[:, ::E] = 0
    else:
        codes = rng.integers(-127, 128, (N, K)).astype(np.int8)
        codes[:, ::E] = 127
    scale16 = (np.abs(rng.standard_normal(N * K // E)) * 0.01 + 1e-3).astype(np.float16)
    if fmt == I8:
        s = scale16.astype(np.float32)          # 11 significant bits: 127 s is exact in fp32
        w = (codes.reshape(N, K // E, E).astype(np.float64) * s.reshape(N, K // E, 1)).reshape(N, K)
        c2, s2 = o.quantize(I8, w.astype(np.float32), N, K)
        assert np.array_equal(c2.reshape(N, K), codes)
        assert np.array_equal(s2, s)
    else:
        aos = o.pack_gguf(fmt, codes, scale16.view(np.uint16), N, K)
        w = o.dequant(fmt, aos, None, N, K)     # exact; fits fp32 exactly
        aos2, _ = o.quantize(fmt, w.astype(np.float32), N, K)
        assert np.array_equal(aos2, aos)


def pin_quant_error_bound(o):
    for fmt in (Q8, Q4, I8):
        _error_bound(o, fmt)


def _error_bound(o, fmt):
    """lq_dequant of the result is within |d| / 2 of the source per element
    (|d| for Q4_0, whose largest positive values clamp at code 15)."""
    N, K = 33, 512
    w = (lqgen.activations(900 + fmt, N * K, np.float32) * 0.03).reshape(N, K)
    q, s = o.quantize(fmt, w, N, K)
    back = o.dequant(fmt, q, s, N, K)
    E = 64 if fmt == I8 else 32
    if fmt == I8:
        d = np.abs(s.astype(np.float64)).reshape(N, K // E, 1)
    else:
        _, sb = o.unpack_gguf(fmt, q, N, K)
        d = np.abs(np.array([o.half_to_double(h) for h in sb.reshape(-1)])).reshape(N, K // E, 1)
    err = np.abs(back - w.astype(np.float64)).reshape(N, K // E, E)
    bound = d * (1.0 if fmt == Q4 else 0.5) * (1 + 1e-6)
    assert np.all(err <= bound)
    # and the bound is not vacuous: some element uses at least 40 % of it
    assert np.max(err / bound) > 0.4


def pin_quant_sources_agree(o):
    for fmt in (Q8, Q4, I8):
        _sources_agree(o, fmt)


def _sources_agree(o, fmt):
    """Values that fp32, fp16 and bf16 all represent exactly (8-bit
    significands, moderate exponents) give identical output."""
    N, K = 5, 128
    rng = np.random.default_rng(11)
    v = (rng.integers(-255, 256, (N, K)) * 2.0 ** rng.integers(-12, -4, (N, K))).astype(np.float32)
    a32 = o.quantize(fmt, v, N, K)
    a16 = o.quantize(fmt, v.astype(np.float16), N, K)
    bf = (v.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bf.astype(np.uint32) << 16).view(np.float32), v)
    ab = o.quantize(fmt, bf, N, K, sdt=lqref.BF16)
    for a in (a16, ab):
        assert np.array_equal(a[0], a32[0])
        if fmt == I8:
            assert np.array_equal(a[1], a32[1])


QUANT_PINS = [pin_quant_hand_blocks, pin_quant_zero_blocks, pin_quant_idempotent, pin_quant_error_bound,
              pin_quant_sources_agree]


@pytest.mark.parametrize("pin", QUANT_PINS, ids=lambda f: f.__name__)
def test_quant_pin(oracle, pin):
    pin(oracle)
