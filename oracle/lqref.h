/*
 * lqref — plain, slow CPU oracle for block-quantized weight x activation
 * products.  TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header, table
 * or helper with the HIP library; it is built by the host compiler alone.
 *
 * What it computes (the plain definition, decoded exactly and summed in fp64):
 *   Q4_0  ("lean" page, model table: GGUF Q4_0 files; "oxinfer" page, "How it
 *          works", quant.rs bullet: two nibbles per byte, f16 scale):
 *          18-byte block = fp16 scale d (little-endian) + 16 code bytes;
 *          byte j holds element j in its low nibble and element j+16 in its
 *          high nibble; w = (q - 8) * d.
 *   Q8_0  ("lean" page: GGUF Q8_0 fixtures): 34-byte block = fp16 scale d +
 *          32 signed int8 codes; w = c * d.
 *   I8B64 ("wgpu-llm" page, "INT8 mode": block size 64): symmetric int8
 *          codes, row-major N x K, one fp32 scale per 64 consecutive codes of
 *          a row; w = c * s.
 *   I8B32 ("oxinfer" page, "How it works": Q8 with 32 weights per scale;
 *          "Pre-quantized checkpoints": int8 codes with fp32 scales): as
 *          I8B64 with one fp32 scale per 32 codes.
 * A matrix is N rows x K columns; blocks run along K; y = W x.
 *
 * Every function returns 0 on success and a negative value on a bad argument.
 * Parity status of each function is listed in the test file that pins it.
 */
#ifndef LQREF_H
#define LQREF_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { LQREF_Q4_0 = 0, LQREF_Q8_0 = 1, LQREF_I8B64 = 2, LQREF_I8B32 = 3 };
enum { LQREF_F32 = 0, LQREF_F16 = 1, LQREF_BF16 = 2 };

/* IEEE binary16 decode (exact in double) and round-to-nearest-even encode. */
double   lqref_half_to_double(uint16_t h);
uint16_t lqref_double_to_half(double v);

/* Weights per block, and bytes of one GGUF block (0 for I8B64 and I8B32,
 * which have no GGUF form). */
int lqref_block_elems(int fmt);
int lqref_gguf_block_bytes(int fmt);

/* Exact decode of a whole matrix into doubles (N*K, row-major).
 * fmt Q4_0/Q8_0: w = GGUF array-of-blocks bytes, scales ignored (may be NULL).
 * fmt I8B64, I8B32: w = int8 codes (N*K), scales = fp32 plane (N*K/64 or
 *                  N*K/32). */
int lqref_dequant(int fmt, const uint8_t* w, const void* scales,
                  int64_t N, int64_t K, double* out);
/* The same value rounded once to fp32 / to fp16 (bit patterns). */
int lqref_dequant_f32(int fmt, const uint8_t* w, const void* scales,
                      int64_t N, int64_t K, float* out);
int lqref_dequant_f16(int fmt, const uint8_t* w, const void* scales,
                      int64_t N, int64_t K, uint16_t* out);

/* GGUF array-of-blocks packer and unpacker (Q4_0, Q8_0 only).
 * codes: N*K int8 (Q4_0: 0..15; Q8_0: -128..127); scales: N*(K/32) fp16 bits. */
int lqref_pack_gguf(int fmt, const int8_t* codes, const uint16_t* scales,
                    int64_t N, int64_t K, uint8_t* out);
int lqref_unpack_gguf(int fmt, const uint8_t* aos, int64_t N, int64_t K,
                      int8_t* codes, uint16_t* scales);

/* Load-time quantization of a row-major N x K matrix ("oxinfer" page, "How
 * it works": block quantization of weights at load time; "wgpu-llm" page,
 * "INT8 mode": symmetric int8, block size 64).  The pages give no rounding
 * rule; the reading implemented here, in IEEE fp32 operations:
 *   Q8_0:  a = max |w| over the 32-block; d = fp16(a / 127);
 *          c = clamp(rint(w / float(d)), -127, 127), 0 when d == 0.
 *   Q4_0:  m = the block's first element of largest |w|; d = fp16(m / -8);
 *          q = clamp(rint(w / float(d)) + 8, 0, 15), 8 when d == 0.
 *   I8B64, I8B32: a = max |w| over the 64- or 32-block; s = a / 127 (fp32);
 *          c = clamp(rint(w / s), -127, 127), 0 when s == 0.
 * rint rounds to nearest, ties to even; fp16() rounds to nearest even.
 * src: N*K values of dtype sdt (LQREF_F32, LQREF_F16 bits, LQREF_BF16 bits),
 * finite.  Q4_0 / Q8_0: out = GGUF array-of-blocks bytes (scales unused);
 * I8B64 / I8B32: out = N*K int8 codes and scales = N*K/64 or N*K/32 fp32. */
int lqref_quantize(int fmt, const void* src, int sdt, int64_t N, int64_t K,
                   uint8_t* out, float* scales);

/* y[i] = sum_k w[rows[i],k] * x[k] and S[i] = sum_k |w[rows[i],k] * x[k]|, in
 * double, k ascending.  x is fp32 (xdt LQREF_F32) or fp16 bits (LQREF_F16).
 * rows == NULL means all N rows (nrows must then equal N).  nthreads >= 1. */
int lqref_gemv(int fmt, const uint8_t* w, const void* scales,
               const void* x, int xdt, int64_t N, int64_t K,
               const int64_t* rows, int64_t nrows,
               double* y, double* S, int nthreads);

/* Y[a,b] = sum_k w[ns[b],k] * X[ms[a],k] and S likewise (Y = X W^T), for the
 * selected token rows ms (nm of them) and weight rows ns (nn of them); output
 * nm x nn row-major.  X is M x K row-major, fp32 or fp16 bits.
 * round_w_f16 = 1 uses RN_fp16(w) in place of w (the fp16 tile contract). */
int lqref_gemm(int fmt, const uint8_t* w, const void* scales,
               const void* X, int xdt, int64_t M, int64_t N, int64_t K,
               const int64_t* ms, int64_t nm, const int64_t* ns, int64_t nn,
               int round_w_f16, double* Y, double* S, int nthreads);

/* Per-matmul activation quantization ("oxinfer" page, "How it works",
 * quant.rs: activations are quantized for each matmul and the decode kernels
 * take integer dot products of int8 activations with the weight codes).  The
 * page gives no rule; the reading here is the page's own Q8 rule (32 values
 * per fp32 scale) applied to each 32-element block of each token row of X
 * (M x K, fp32 or fp16 bits), in IEEE fp32 operations:
 *   a = max |x| over the block; s = a / 127 (fp32);
 *   q = clamp(rint(x / s), -127, 127) (rint: nearest, ties to even), 0 when s == 0;
 *   sum = the block's sum of q (int32).
 * Outputs: q (M*K int8), s (M*K/32 fp32), sum (M*K/32 int32). */
int lqref_quantize_act(const void* X, int xdt, int64_t M, int64_t K,
                       int8_t* q, float* s, int32_t* sum);

/* Integer-dot product on quantized activations (q, s as above):
 *   Y[m,n] = sum_b  ws(n,b) * s[m,b] * I(m,n,b),
 *   I(m,n,b) = sum over the 32 elements k of block b of c(n,k) * q[m,k],
 * where c is the weight's integer code (q - 8 for Q4_0, the int8 code
 * otherwise) and ws(n,b) the scale of the weight block holding block b (fp16
 * d, or the fp32 scale; an int8 block-64 scale covers two blocks).  I is
 * exact; the sum over b is in double.  S[m,n] = sum_b |ws s I|.  Output M x N
 * row-major; K a multiple of the weight block. */
int lqref_gemv_q8act(int fmt, const uint8_t* w, const void* scales,
                     const int8_t* q, const float* s, int64_t M, int64_t N, int64_t K,
                     double* Y, double* S, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
