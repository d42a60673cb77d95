"""Plant plausible mistakes in copies of the CPU oracle and check that the pins
catch every one.  Runs on the CPU only: each mutant is a g++ build of the
oracle source with one textual change, loaded from a temporary directory.
"""
import pytest

from oracle import lqref
from tests.test_oracle_pins import ALL_PINS
from tests.test_oracle_quant import QUANT_PINS
from tests.test_oracle_q8act import Q8ACT_PINS

MUTANTS = {
    # nibble order (2j, 2j+1) instead of (j, j+16)
    "nibble_order": ("out[j] = static_cast<double>(lo - 8) * d;\n        out[j + 16] = static_cast<double>(hi - 8) * d;",
                     "out[2 * j] = static_cast<double>(lo - 8) * d;\n        out[2 * j + 1] = static_cast<double>(hi - 8) * d;"),
    # the -8 offset dropped from the low nibble
    "drop_offset": ("out[j] = static_cast<double>(lo - 8) * d;", "out[j] = static_cast<double>(lo) * d;"),
    # fp16 exponent bias off by one
    "half_bias": ("std::ldexp(static_cast<double>(1024 + m), e - 25)", "std::ldexp(static_cast<double>(1024 + m), e - 24)"),
    # fp16 subnormal scale wrong
    "half_subnormal": ("std::ldexp(static_cast<double>(m), -24)", "std::ldexp(static_cast<double>(m), -25)"),
    # Q8_0 codes read as unsigned
    "q8_unsigned": ("const int c = static_cast<int8_t>(b[2 + j]);", "const int c = b[2 + j];"),
    # scale bytes read big-endian
    "scale_endianness": ("const double d = half_to_double(static_cast<uint16_t>(b[0] | (b[1] << 8)));\n    for (int j = 0; j < 16; ++j)",
                         "const double d = half_to_double(static_cast<uint16_t>((b[0] << 8) | b[1]));\n    for (int j = 0; j < 16; ++j)"),
    # int8 scale index using 32-wide blocks whatever the block size
    "i8_scale_index": ("static_cast<double>(s[k / E])", "static_cast<double>(s[k / 32 % (K / E)])"),
    # S without the absolute value
    "abs_dropped": ("abs_acc += std::fabs(p);\n        }\n        y[i] = acc;", "abs_acc += p;\n        }\n        y[i] = acc;"),
    # GEMM reads X transposed
    "gemm_transposed_x": ("x_at(X, xdt, ms[a] * K + k)", "x_at(X, xdt, k * M + ms[a])"),
    # fp16 encoder rounds ties up instead of to even
    "ties_up": ("return (std::fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl + 1.0;"),
    # fp16 tile of the fp32-scale formats rounded through fp32 first (double rounding)
    "f16_via_f32": ("for (int64_t k = 0; k < K; ++k) out[n * K + k] = double_to_half(row[k]);",
                    "for (int64_t k = 0; k < K; ++k) out[n * K + k] = double_to_half(static_cast<float>(row[k]));"),
    # GEMM ignores the fp16 tile rounding flag
    "gemm_no_f16_round": ("if (round_w_f16)", "if (false && round_w_f16)"),
    # quantizer: ties rounded away from zero instead of to even
    "quant_round_away": ("const float r = std::nearbyint(v);", "const float r = std::round(v);"),
    # quantizer: Q4_0 scale from the magnitude, sign dropped
    "quant_q4_unsigned": ("m = std::fabs(w[e]) > std::fabs(m) ? w[e] : m;", "m = std::fabs(w[e]) > std::fabs(m) ? std::fabs(w[e]) : m;"),
    # quantizer: Q4_0 takes the last element of largest magnitude
    "quant_q4_last_tie": ("m = std::fabs(w[e]) > std::fabs(m) ? w[e] : m;", "m = std::fabs(w[e]) >= std::fabs(m) ? w[e] : m;"),
    # quantizer: Q8_0 divides by 128
    "quant_q8_divisor": ("d16 = double_to_half(double(a / 127.0f));", "d16 = double_to_half(double(a / 128.0f));"),
    # quantizer: int8 block-64 maximum over the first half of the block only
    "quant_i8_half_block": ("for (int e = 0; e < E; ++e) a = std::fabs(w[e]) > a ? std::fabs(w[e]) : a;\n                const float s",
                            "for (int e = 0; e < 32; ++e) a = std::fabs(w[e]) > a ? std::fabs(w[e]) : a;\n                const float s"),
    # activation quantizer: divisor 128
    "act_divisor": ("const float sc = a / 127.0f;", "const float sc = a / 128.0f;"),
    # activation quantizer: block sum of |q|
    "act_sum_abs": ("            t += c;", "            t += c < 0 ? -c : c;"),
    # activation quantizer: the largest element from the first half block only
    "act_half_block": ("for (int e = 0; e < 32; ++e) a = std::fabs(x[e]) > a ? std::fabs(x[e]) : a;\n            const float sc",
                       "for (int e = 0; e < 16; ++e) a = std::fabs(x[e]) > a ? std::fabs(x[e]) : a;\n            const float sc"),
    # integer-dot product: Q4_0 offset dropped
    "q8act_q4_offset": ("(blk[2 + j - 16] >> 4)) - 8;", "(blk[2 + j - 16] >> 4));"),
    # integer-dot product: high nibble read as the low one
    "q8act_high_nibble": ("(blk[2 + j - 16] >> 4)) - 8;", "(blk[2 + j - 16] & 0x0F)) - 8;"),
    # integer-dot product: int8 block-64 scale indexed per 32 elements
    "q8act_i8_scale_index": ("*scale = static_cast<const float*>(scales)[n * (K / E) + k / E];",
                             "*scale = static_cast<const float*>(scales)[n * (K / E) + (k / 32) % (K / E)];"),
    # integer-dot product: every token uses token 0's codes
    "q8act_token_row": ("I += int64_t(c) * int64_t(q[m * K + b * 32 + e]);", "I += int64_t(c) * int64_t(q[b * 32 + e]);"),
    # integer-dot product: S without the absolute value
    "q8act_abs": ("abs_acc += std::fabs(t);\n            }\n            Y[m * N + n] = acc;",
                  "abs_acc += t;\n            }\n            Y[m * N + n] = acc;"),
    # quantizer: bf16 widened with the wrong shift
    "quant_bf16_shift": ("uint32_t bits = uint32_t(h) << 16;", "uint32_t bits = uint32_t(h) << 15;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = lqref.source_text()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutant = lqref.build_variant(src.replace(old, new), str(tmp_path))
    failed = []
    for pin in ALL_PINS + QUANT_PINS + Q8ACT_PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
