// lqref — plain CPU oracle (test infrastructure only; see lqref.h).
//
// Written for a reader checking it against the block definitions by eye:
// every block is decoded exactly into doubles, and every sum is an ordinary
// k-ascending loop in double.  No blocking, fusion or reordering.  Threads
// only split the list of output rows; each row is summed by one thread.
#include "lqref.h"

#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// ---------------------------------------------------------------------------
// IEEE 754 binary16.  Field layout: 1 sign bit, 5 exponent bits (bias 15),
// 10 fraction bits.  The fp16 scales of Q4_0 / Q8_0 ("oxinfer" page, "How it
// works": "f16 scale") are decoded with this.
// ---------------------------------------------------------------------------
double half_to_double(uint16_t h) {
    const int s = h >> 15;
    const int e = (h >> 10) & 31;
    const int m = h & 1023;
    double v;
    if (e == 0) {
        v = std::ldexp(static_cast<double>(m), -24);          // zero / subnormal
    } else if (e == 31) {
        v = (m == 0) ? INFINITY : NAN;                        // inf / NaN
    } else {
        v = std::ldexp(static_cast<double>(1024 + m), e - 25);  // normal
    }
    return s ? -v : v;
}

// Round a non-negative finite double n to the nearest integer, ties to even.
double round_half_even(double n) {
    const double fl = std::floor(n);
    const double r = n - fl;  // exact: n and fl are within one binade of 2^52
    if (r > 0.5) return fl + 1.0;
    if (r < 0.5) return fl;
    return (std::fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

uint16_t double_to_half(double v) {
    const uint16_t sign = std::signbit(v) ? 0x8000 : 0;
    if (std::isnan(v)) return sign | 0x7E00;                  // quiet NaN
    const double a = std::fabs(v);
    // 65520 is halfway between 65504 (largest finite, odd fraction) and
    // 2^16; ties go to the even neighbour, which is out of range -> inf.
    if (a >= 65520.0) return sign | 0x7C00;
    if (a < std::ldexp(1.0, -14)) {
        // Subnormal range: value = m * 2^-24, m in [0, 1024].  m == 1024 is
        // the smallest normal, whose bit pattern is also 1024.
        const double m = round_half_even(a / std::ldexp(1.0, -24));
        return sign | static_cast<uint16_t>(m);
    }
    int E;
    std::frexp(a, &E);            // a = f * 2^E, f in [0.5, 1)
    int e = E - 1;                // a in [2^e, 2^(e+1))
    double m = round_half_even(a / std::ldexp(1.0, e - 10));  // in [1024, 2048]
    if (m == 2048.0) { m = 1024.0; e += 1; }
    if (e + 15 >= 31) return sign | 0x7C00;
    return sign | static_cast<uint16_t>(((e + 15) << 10) | (static_cast<int>(m) - 1024));
}

int block_elems(int fmt) {
    switch (fmt) {
        case LQREF_Q4_0: return 32;
        case LQREF_Q8_0: return 32;
        case LQREF_I8B64: return 64;
        case LQREF_I8B32: return 32;
        default: return 0;
    }
}

int gguf_block_bytes(int fmt) {
    switch (fmt) {
        case LQREF_Q4_0: return 2 + 16;   // fp16 d + 32 nibbles
        case LQREF_Q8_0: return 2 + 32;   // fp16 d + 32 int8
        default: return 0;
    }
}

// The int8 formats with fp32 scales are stored as two planes (codes, scales)
// instead of GGUF blocks.
bool planar(int fmt) { return fmt == LQREF_I8B64 || fmt == LQREF_I8B32; }

bool shape_ok(int fmt, int64_t N, int64_t K) {
    const int be = block_elems(fmt);
    return be > 0 && N >= 0 && K >= 0 && (K % be) == 0;
}

// Q4_0 block: bytes 0-1 = d (little-endian fp16); byte 2+j (j = 0..15) holds
// element j in its low nibble and element j+16 in its high nibble (the GGUF
// order); w = (q - 8) * d, exact in double (a 4-bit integer times an fp16).
void decode_q4_0_block(const uint8_t* b, double out[32]) {
    const double d = half_to_double(static_cast<uint16_t>(b[0] | (b[1] << 8)));
    for (int j = 0; j < 16; ++j) {
        const int lo = b[2 + j] & 0x0F;
        const int hi = b[2 + j] >> 4;
        out[j] = static_cast<double>(lo - 8) * d;
        out[j + 16] = static_cast<double>(hi - 8) * d;
    }
}

// Q8_0 block: bytes 0-1 = d (little-endian fp16); bytes 2..33 = 32 int8
// codes in element order; w = c * d, exact in double.
void decode_q8_0_block(const uint8_t* b, double out[32]) {
    const double d = half_to_double(static_cast<uint16_t>(b[0] | (b[1] << 8)));
    for (int j = 0; j < 32; ++j) {
        const int c = static_cast<int8_t>(b[2 + j]);
        out[j] = static_cast<double>(c) * d;
    }
}

// Decode row n of a matrix into out[0..K).
void decode_row(int fmt, const uint8_t* w, const void* scales, int64_t K,
                int64_t n, double* out) {
    if (planar(fmt)) {
        // I8B64 / I8B32: codes row-major N x K; one fp32 scale per E = 64 or
        // 32 codes of a row; w = c * s, exact in double (8-bit times 24-bit
        // significand).
        const int64_t E = block_elems(fmt);
        const int8_t* c = reinterpret_cast<const int8_t*>(w) + n * K;
        const float* s = static_cast<const float*>(scales) + n * (K / E);
        for (int64_t k = 0; k < K; ++k)
            out[k] = static_cast<double>(c[k]) * static_cast<double>(s[k / E]);
        return;
    }
    const int64_t nb = K / 32;
    const int bb = gguf_block_bytes(fmt);
    const uint8_t* row = w + n * nb * bb;
    for (int64_t b = 0; b < nb; ++b) {
        if (fmt == LQREF_Q4_0) decode_q4_0_block(row + b * bb, out + b * 32);
        else decode_q8_0_block(row + b * bb, out + b * 32);
    }
}

double x_at(const void* x, int xdt, int64_t i) {
    if (xdt == LQREF_F32) return static_cast<double>(static_cast<const float*>(x)[i]);
    return half_to_double(static_cast<const uint16_t*>(x)[i]);
}

// Run fn(i) for i in [0, n) on up to nthreads threads (contiguous chunks).
template <class F>
void parallel_for(int64_t n, int nthreads, F fn) {
    if (nthreads < 1) nthreads = 1;
    if (n < nthreads) nthreads = static_cast<int>(n > 0 ? n : 1);
    if (nthreads == 1) {
        for (int64_t i = 0; i < n; ++i) fn(i);
        return;
    }
    std::vector<std::thread> ts;
    const int64_t chunk = (n + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        const int64_t lo = t * chunk;
        const int64_t hi = std::min<int64_t>(n, lo + chunk);
        if (lo >= hi) break;
        ts.emplace_back([lo, hi, &fn] {
            for (int64_t i = lo; i < hi; ++i) fn(i);
        });
    }
    for (auto& th : ts) th.join();
}

}  // namespace

extern "C" {

double lqref_half_to_double(uint16_t h) { return half_to_double(h); }
uint16_t lqref_double_to_half(double v) { return double_to_half(v); }
int lqref_block_elems(int fmt) { return block_elems(fmt); }
int lqref_gguf_block_bytes(int fmt) { return gguf_block_bytes(fmt); }

int lqref_dequant(int fmt, const uint8_t* w, const void* scales, int64_t N,
                  int64_t K, double* out) {
    if (!shape_ok(fmt, N, K) || !w || !out) return -1;
    if (planar(fmt) && !scales) return -1;
    for (int64_t n = 0; n < N; ++n) decode_row(fmt, w, scales, K, n, out + n * K);
    return 0;
}

int lqref_dequant_f32(int fmt, const uint8_t* w, const void* scales, int64_t N,
                      int64_t K, float* out) {
    if (!shape_ok(fmt, N, K) || !w || !out) return -1;
    if (planar(fmt) && !scales) return -1;
    std::vector<double> row(static_cast<size_t>(K));
    for (int64_t n = 0; n < N; ++n) {
        decode_row(fmt, w, scales, K, n, row.data());
        // One IEEE round-to-nearest-even conversion double -> float.
        for (int64_t k = 0; k < K; ++k) out[n * K + k] = static_cast<float>(row[k]);
    }
    return 0;
}

int lqref_dequant_f16(int fmt, const uint8_t* w, const void* scales, int64_t N,
                      int64_t K, uint16_t* out) {
    if (!shape_ok(fmt, N, K) || !w || !out) return -1;
    if (planar(fmt) && !scales) return -1;
    std::vector<double> row(static_cast<size_t>(K));
    for (int64_t n = 0; n < N; ++n) {
        decode_row(fmt, w, scales, K, n, row.data());
        for (int64_t k = 0; k < K; ++k) out[n * K + k] = double_to_half(row[k]);
    }
    return 0;
}

int lqref_pack_gguf(int fmt, const int8_t* codes, const uint16_t* scales,
                    int64_t N, int64_t K, uint8_t* out) {
    if ((fmt != LQREF_Q4_0 && fmt != LQREF_Q8_0) || !shape_ok(fmt, N, K)) return -1;
    if (!codes || !scales || !out) return -1;
    const int64_t nb = K / 32;
    const int bb = gguf_block_bytes(fmt);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < nb; ++b) {
            uint8_t* blk = out + (n * nb + b) * bb;
            const uint16_t d = scales[n * nb + b];
            blk[0] = static_cast<uint8_t>(d & 0xFF);
            blk[1] = static_cast<uint8_t>(d >> 8);
            const int8_t* c = codes + n * K + b * 32;
            if (fmt == LQREF_Q4_0) {
                for (int j = 0; j < 16; ++j) {
                    if (c[j] < 0 || c[j] > 15 || c[j + 16] < 0 || c[j + 16] > 15) return -2;
                    blk[2 + j] = static_cast<uint8_t>(c[j] | (c[j + 16] << 4));
                }
            } else {
                for (int j = 0; j < 32; ++j) blk[2 + j] = static_cast<uint8_t>(c[j]);
            }
        }
    }
    return 0;
}

int lqref_unpack_gguf(int fmt, const uint8_t* aos, int64_t N, int64_t K,
                      int8_t* codes, uint16_t* scales) {
    if ((fmt != LQREF_Q4_0 && fmt != LQREF_Q8_0) || !shape_ok(fmt, N, K)) return -1;
    if (!aos || !codes || !scales) return -1;
    const int64_t nb = K / 32;
    const int bb = gguf_block_bytes(fmt);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t* blk = aos + (n * nb + b) * bb;
            scales[n * nb + b] = static_cast<uint16_t>(blk[0] | (blk[1] << 8));
            int8_t* c = codes + n * K + b * 32;
            if (fmt == LQREF_Q4_0) {
                for (int j = 0; j < 16; ++j) {
                    c[j] = static_cast<int8_t>(blk[2 + j] & 0x0F);
                    c[j + 16] = static_cast<int8_t>(blk[2 + j] >> 4);
                }
            } else {
                for (int j = 0; j < 32; ++j) c[j] = static_cast<int8_t>(blk[2 + j]);
            }
        }
    }
    return 0;
}

// Source element i as a float (exact for all three source types).
static float source_at(const void* src, int sdt, int64_t i) {
    if (sdt == LQREF_F32) return static_cast<const float*>(src)[i];
    const uint16_t h = static_cast<const uint16_t*>(src)[i];
    if (sdt == LQREF_F16) return static_cast<float>(half_to_double(h));
    uint32_t bits = uint32_t(h) << 16;   // bf16 is the top half of an fp32
    float f;
    std::memcpy(&f, &bits, sizeof f);
    return f;
}

// Round to the nearest integer, ties to even, then clamp (the value is finite).
static int round_clamp(float v, int lo, int hi) {
    const float r = std::nearbyint(v);   // default rounding mode: nearest even
    if (r < float(lo)) return lo;
    if (r > float(hi)) return hi;
    return int(r);
}

int lqref_quantize(int fmt, const void* src, int sdt, int64_t N, int64_t K,
                   uint8_t* out, float* scales) {
    if (!shape_ok(fmt, N, K) || !src || !out) return -1;
    if (sdt != LQREF_F32 && sdt != LQREF_F16 && sdt != LQREF_BF16) return -1;
    if (planar(fmt) && !scales) return -1;
    const int E = block_elems(fmt);
    const int64_t nb = K / E;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < nb; ++b) {
            float w[64];
            for (int e = 0; e < E; ++e) w[e] = source_at(src, sdt, n * K + b * E + e);
            if (planar(fmt)) {
                float a = 0.0f;
                for (int e = 0; e < E; ++e) a = std::fabs(w[e]) > a ? std::fabs(w[e]) : a;
                const float s = a / 127.0f;
                scales[n * nb + b] = s;
                int8_t* c = reinterpret_cast<int8_t*>(out) + n * K + b * E;
                for (int e = 0; e < E; ++e) c[e] = int8_t(s == 0.0f ? 0 : round_clamp(w[e] / s, -127, 127));
                continue;
            }
            uint8_t* blk = out + (n * nb + b) * gguf_block_bytes(fmt);
            uint16_t d16;
            if (fmt == LQREF_Q8_0) {
                float a = 0.0f;
                for (int e = 0; e < 32; ++e) a = std::fabs(w[e]) > a ? std::fabs(w[e]) : a;
                d16 = double_to_half(double(a / 127.0f));
            } else {
                float m = 0.0f;   // first element of largest magnitude, with its sign
                for (int e = 0; e < 32; ++e) m = std::fabs(w[e]) > std::fabs(m) ? w[e] : m;
                d16 = double_to_half(double(m / -8.0f));
            }
            blk[0] = uint8_t(d16 & 0xFF);
            blk[1] = uint8_t(d16 >> 8);
            const float d = float(half_to_double(d16));
            int q[32];
            for (int e = 0; e < 32; ++e) {
                if (fmt == LQREF_Q8_0) q[e] = d == 0.0f ? 0 : round_clamp(w[e] / d, -127, 127);
                else q[e] = d == 0.0f ? 8 : round_clamp(w[e] / d, -8, 7) + 8;
            }
            if (fmt == LQREF_Q8_0) {
                for (int j = 0; j < 32; ++j) blk[2 + j] = uint8_t(int8_t(q[j]));
            } else {
                for (int j = 0; j < 16; ++j) blk[2 + j] = uint8_t(q[j] | (q[j + 16] << 4));
            }
        }
    }
    return 0;
}

int lqref_quantize_act(const void* X, int xdt, int64_t M, int64_t K,
                       int8_t* q, float* s, int32_t* sum) {
    if (!X || !q || !s || !sum || M < 0 || K < 0 || K % 32 != 0) return -1;
    if (xdt != LQREF_F32 && xdt != LQREF_F16) return -1;
    const int64_t nb = K / 32;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t b = 0; b < nb; ++b) {
            float x[32];
            for (int e = 0; e < 32; ++e) x[e] = source_at(X, xdt, m * K + b * 32 + e);
            float a = 0.0f;
            for (int e = 0; e < 32; ++e) a = std::fabs(x[e]) > a ? std::fabs(x[e]) : a;
            const float sc = a / 127.0f;
            int32_t t = 0;
            for (int e = 0; e < 32; ++e) {
                const int c = sc == 0.0f ? 0 : round_clamp(x[e] / sc, -127, 127);
                q[m * K + b * 32 + e] = int8_t(c);
                t += c;
            }
            s[m * nb + b] = sc;
            sum[m * nb + b] = t;
        }
    }
    return 0;
}

// Integer code and scale of the weight block of row n that holds element k:
// Q4_0 q - 8 with the fp16 d, Q8_0 the int8 code with the fp16 d, the int8
// formats the code with the fp32 scale of its 64- or 32-block.
static void code_and_scale(int fmt, const uint8_t* w, const void* scales, int64_t K, int64_t n, int64_t k,
                           int* code, double* scale) {
    if (planar(fmt)) {
        const int64_t E = block_elems(fmt);
        *code = reinterpret_cast<const int8_t*>(w)[n * K + k];
        *scale = static_cast<const float*>(scales)[n * (K / E) + k / E];
        return;
    }
    const int bb = gguf_block_bytes(fmt);
    const uint8_t* blk = w + (n * (K / 32) + k / 32) * bb;
    *scale = half_to_double(static_cast<uint16_t>(blk[0] | (blk[1] << 8)));
    const int j = int(k % 32);
    if (fmt == LQREF_Q4_0) *code = (j < 16 ? (blk[2 + j] & 0x0F) : (blk[2 + j - 16] >> 4)) - 8;
    else *code = static_cast<int8_t>(blk[2 + j]);
}

int lqref_gemv_q8act(int fmt, const uint8_t* w, const void* scales,
                     const int8_t* q, const float* s, int64_t M, int64_t N, int64_t K,
                     double* Y, double* S, int nthreads) {
    if (!shape_ok(fmt, N, K) || !w || !q || !s || !Y || !S || M < 0) return -1;
    if (planar(fmt) && !scales) return -1;
    const int64_t nb = K / 32;
    parallel_for(N, nthreads, [&](int64_t n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, abs_acc = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                int64_t I = 0;
                double ws = 0.0;
                for (int e = 0; e < 32; ++e) {
                    int c;
                    code_and_scale(fmt, w, scales, K, n, b * 32 + e, &c, &ws);
                    I += int64_t(c) * int64_t(q[m * K + b * 32 + e]);
                }
                const double t = ws * static_cast<double>(s[m * nb + b]) * static_cast<double>(I);
                acc += t;
                abs_acc += std::fabs(t);
            }
            Y[m * N + n] = acc;
            S[m * N + n] = abs_acc;
        }
    });
    return 0;
}

int lqref_gemv(int fmt, const uint8_t* w, const void* scales, const void* x,
               int xdt, int64_t N, int64_t K, const int64_t* rows, int64_t nrows,
               double* y, double* S, int nthreads) {
    if (!shape_ok(fmt, N, K) || !w || !x || !y || !S) return -1;
    if (planar(fmt) && !scales) return -1;
    if (xdt != LQREF_F32 && xdt != LQREF_F16) return -1;
    if (!rows && nrows != N) return -1;
    if (rows) {
        for (int64_t i = 0; i < nrows; ++i)
            if (rows[i] < 0 || rows[i] >= N) return -1;
    }
    std::vector<double> xd(static_cast<size_t>(K));
    for (int64_t k = 0; k < K; ++k) xd[k] = x_at(x, xdt, k);  // exact widening
    parallel_for(nrows, nthreads, [&](int64_t i) {
        const int64_t n = rows ? rows[i] : i;
        std::vector<double> wr(static_cast<size_t>(K));
        decode_row(fmt, w, scales, K, n, wr.data());
        double acc = 0.0, abs_acc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double p = wr[k] * xd[k];
            acc += p;
            abs_acc += std::fabs(p);
        }
        y[i] = acc;
        S[i] = abs_acc;
    });
    return 0;
}

int lqref_gemm(int fmt, const uint8_t* w, const void* scales, const void* X,
               int xdt, int64_t M, int64_t N, int64_t K, const int64_t* ms,
               int64_t nm, const int64_t* ns, int64_t nn, int round_w_f16,
               double* Y, double* S, int nthreads) {
    if (!shape_ok(fmt, N, K) || M < 0 || !w || !X || !Y || !S || !ms || !ns) return -1;
    if (planar(fmt) && !scales) return -1;
    if (xdt != LQREF_F32 && xdt != LQREF_F16) return -1;
    for (int64_t a = 0; a < nm; ++a) if (ms[a] < 0 || ms[a] >= M) return -1;
    for (int64_t b = 0; b < nn; ++b) if (ns[b] < 0 || ns[b] >= N) return -1;
    // Selected token rows of X, widened exactly to double.
    std::vector<double> xd(static_cast<size_t>(nm * K));
    for (int64_t a = 0; a < nm; ++a)
        for (int64_t k = 0; k < K; ++k) xd[a * K + k] = x_at(X, xdt, ms[a] * K + k);
    parallel_for(nn, nthreads, [&](int64_t b) {
        std::vector<double> wr(static_cast<size_t>(K));
        decode_row(fmt, w, scales, K, ns[b], wr.data());
        if (round_w_f16)
            for (int64_t k = 0; k < K; ++k) wr[k] = half_to_double(double_to_half(wr[k]));
        for (int64_t a = 0; a < nm; ++a) {
            const double* xr = xd.data() + a * K;
            double acc = 0.0, abs_acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double p = wr[k] * xr[k];
                acc += p;
                abs_acc += std::fabs(p);
            }
            Y[a * nn + b] = acc;
            S[a * nn + b] = abs_acc;
        }
    });
    return 0;
}

}  // extern "C"
