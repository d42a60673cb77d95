/*
 * lq.h — C ABI of liblq: block-quantized weight x activation products on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation.  A weight matrix W has N rows and K columns and is stored in
 * blocks that run along K.  The library computes y = W x for one token (a
 * dequantizing matrix-vector product, the decode step) and Y = X W^T for a
 * chunk of M tokens (the prefill matrix product).  "Decode is memory-bandwidth
 * bound: every generated token streams all dense weights once", while prefill
 * is compute-bound ("oxinfer" page, "Performance"); prefill GPU kernels
 * dequantize weights into on-chip memory and run a dense tile ("oxinfer" page,
 * "Platforms and accelerators" and "Browser (WebGPU)").
 *
 * Weight formats (enum lq_fmt):
 *   LQ_Q4_0   GGUF Q4_0 ("lean" page, model table; "oxinfer" page, "How it
 *             works": two nibbles per byte, f16 scale).  32 weights per block,
 *             one fp16 scale d, 4-bit codes q; w = (q - 8) * d.  Within a
 *             block's 16 code bytes, byte j holds element j in its low nibble
 *             and element j + 16 in its high nibble (the GGUF order).
 *   LQ_Q8_0   GGUF Q8_0 ("lean" page, Q8_0 parity fixtures).  32 int8 codes c
 *             and one fp16 scale d per block; w = c * d.
 *   LQ_I8B64  symmetric int8 with block size 64 ("wgpu-llm" page, "INT8
 *             mode", --block-size 64).  int8 codes c, one fp32 scale s per 64
 *             consecutive codes of a row; w = c * s (no zero point).
 *   LQ_I8B32  the "oxinfer" page's Q8 ("How it works": 32 weights per scale;
 *             "Pre-quantized checkpoints": int8 codes X.q8 with fp32 scales
 *             X.q8s).  int8 codes c, one fp32 scale s per 32 consecutive
 *             codes of a row; w = c * s.  Every call treats it as LQ_I8B64
 *             with 32-code blocks.
 *
 * Packed layout (what every W argument points to).  Like the split layout in
 * which the "oxinfer" page stores quantized matrices ("Pre-quantized
 * checkpoints": codes and scales as separate tensors, in the kernels'
 * in-memory layout), a packed matrix is a code plane followed by a scale
 * plane, both in the order the GPU kernels read them.
 *   A unit is one scale block of one row: 32 weights (LQ_Q4_0, LQ_Q8_0,
 *   LQ_I8B32) or 64 (LQ_I8B64), with nu = K / (unit weights) units per row.
 *   Its codes are P parts of 16 bytes: P = 1 (Q4_0: 16 bytes in GGUF byte
 *   order), 2 (Q8_0, LQ_I8B32: 32 int8) or 4 (LQ_I8B64: 64 int8); part p
 *   holds the unit's code bytes 16p .. 16p + 15.  Its scale is fp16 (Q4_0,
 *   Q8_0) or fp32 (LQ_I8B64, LQ_I8B32).
 *   Rows are grouped in tiles of 64: tile t holds rows 64t .. 64t + nr - 1
 *   with nr = min(64, N - 64t).  For row n = 64t + r and unit u:
 *     code part p at byte   16 * (64 t nu P + (u P + p) nr + r)
 *     scale at element      64 t nu + u nr + r   of the scale plane
 *   (inside a tile: unit-major, then part, then row), so part p of unit u
 *   for all rows of a tile is one contiguous run of nr * 16 bytes.  The
 *   code plane is N K / 2 bytes (Q4_0) or N K bytes; the scale plane starts
 *   at lq_scale_offset(), the code-plane size rounded up to 256 bytes.  The
 *   weight bytes equal those of the GGUF form (18 or 34 bytes per 32
 *   weights; 68 bytes per 64 for LQ_I8B64, 36 per 32 for LQ_I8B32) plus at
 *   most 255 bytes of
 *   padding between the planes (left as allocated).
 *
 * Conventions for every call.
 *   - Pointers named W, x, X, y, Y, out, dst, src, codes, scales, ws are
 *     DEVICE pointers (memory the caller allocated on the current HIP device);
 *     `descs` of the batch calls is a HOST pointer.  The caller owns every
 *     buffer and the library borrows them for the call, as the "oxinfer"
 *     page's loader borrows quantized weights in place ("Pre-quantized
 *     checkpoints": QBuf, no copy); it keeps no pointer after a call returns
 *     and allocates no device memory.
 *   - Workspaces.  Calls that may split K across workgroups take an optional
 *     `ws` / `ws_bytes`: the GEMV calls (lq_gemv_workspace_bytes() bytes,
 *     any contents: no clearing needed, every call leaves it reusable; without
 *     one a GEMV keeps each tile's K inside one workgroup, which is correct
 *     but slower for matrices of few rows) and the GEMM calls
 *     (lq_gemm_workspace_bytes()).  Calls that run at the same time on
 *     different streams need workspaces of their own; calls on one stream may
 *     share one.
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *     Calls only enqueue work (no implicit synchronisation); results are
 *     ready when the stream reaches that point.
 *   - Sizes are int64_t: N, K, M >= 1; N <= 2^31 - 1, M <= 2^31 - 1,
 *     K <= 2^25.  K must be a multiple of the format's block (32, 32, 64, 32).
 *   - Alignment: W, x, X, dst, out and codes must be 16-byte aligned; y, Y
 *     and scales 4-byte aligned; src (GGUF bytes) 2-byte aligned.
 *   - Activations: x / X are fp32 (LQ_F32) or fp16 (LQ_F16), contiguous; X is
 *     M x K row-major (token-major).  Outputs y / Y are always fp32.
 *   - Output buffers must not overlap inputs (undefined behaviour, unchecked).
 *   - Errors: every call returns an lq_status.  All argument checks happen
 *     before any HIP call, so a rejected call touches no device state.  On a
 *     failure lq_last_error() returns a message for the calling thread.
 *     Nothing aborts, prints or throws across the ABI.
 *   - Thread safety: the library holds no state besides a per-device record
 *     of compute-unit counts and a counter of launch tags, both guarded, so
 *     calls may come from several host threads on several streams.  Calls
 *     that write the same buffers (outputs, workspaces) must be ordered by
 *     the caller.
 */
#ifndef LQ_H
#define LQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LQ_ABI_VERSION 8

typedef enum lq_fmt { LQ_Q4_0 = 0, LQ_Q8_0 = 1, LQ_I8B64 = 2, LQ_I8B32 = 3 } lq_fmt;
/* Activation and source dtypes.  LQ_BF16 is accepted only as the source of
 * lq_quantize. */
typedef enum lq_dtype { LQ_F32 = 0, LQ_F16 = 1, LQ_BF16 = 2 } lq_dtype;

typedef enum lq_status {
    LQ_OK = 0,
    LQ_ERR_ARG = 1,          /* null pointer, bad count, bad enum-like value */
    LQ_ERR_SHAPE = 2,        /* N, K or M out of range, K not a block multiple */
    LQ_ERR_ALIGN = 3,        /* a pointer misses its required alignment */
    LQ_ERR_FMT = 4,          /* unknown format, or format not valid for the call */
    LQ_ERR_DTYPE = 5,        /* unknown activation dtype */
    LQ_ERR_UNSUPPORTED = 6,  /* valid combination this version does not implement */
    LQ_ERR_WORKSPACE = 7,    /* workspace missing or smaller than required */
    LQ_ERR_HIP = 8           /* no HIP device, or a HIP runtime call failed */
} lq_status;

/* Returns LQ_ABI_VERSION. */
int32_t lq_abi_version(void);

/* Checks that a HIP device is present and caches its properties.  Returns
 * LQ_ERR_HIP (with a message) when there is none.  Other calls initialise on
 * first use; calling this first is optional. */
lq_status lq_init(void);

/* Weights per block of `fmt` (32, 32, 64, 32); 0 for an unknown format. */
int32_t lq_block_elems(int32_t fmt);

/* Bytes of the packed layout above for an N x K matrix; 0 if fmt, N or K is
 * invalid. */
size_t lq_packed_bytes(int32_t fmt, int64_t N, int64_t K);

/* Offset of the scale plane inside the packed layout; 0 if invalid. */
size_t lq_scale_offset(int32_t fmt, int64_t N, int64_t K);

/* Bytes of the GGUF array-of-blocks form (18 or 34 bytes per block); 0 for
 * LQ_I8B64 and LQ_I8B32 (no GGUF form) or invalid arguments. */
size_t lq_gguf_bytes(int32_t fmt, int64_t N, int64_t K);

/* GGUF array-of-blocks -> packed layout (a byte permutation, no arithmetic).
 * src: N*K/32 GGUF blocks, each the fp16 scale (little-endian) followed by
 * the codes, as a GGUF reader holds them ("lean" page: the engine reads
 * quantized GGUF files).  dst: lq_packed_bytes() bytes.  LQ_I8B64 and
 * LQ_I8B32 return LQ_ERR_FMT: they have no GGUF form (use lq_pack_planes). */
lq_status lq_repack_gguf(int32_t fmt, const void* src, void* dst,
                         int64_t N, int64_t K, void* stream);

/* Row-major code and scale planes -> packed layout (a byte permutation).
 * codes: the units' code bytes row by row, unit by unit (N * K / 2 bytes for
 * Q4_0 in GGUF byte order, N * K int8 otherwise); scales: one per unit in
 * the same order, N * K / 32 fp16 (Q4_0, Q8_0), N * K / 64 fp32 (LQ_I8B64)
 * or N * K / 32 fp32 (LQ_I8B32).  This is the "oxinfer" page's split form ("Pre-quantized
 * checkpoints": X.q4 + X.q4s, X.q8 + X.q8s). */
lq_status lq_pack_planes(int32_t fmt, const void* codes, const void* scales,
                         void* dst, int64_t N, int64_t K, void* stream);

/* Unpacked weights: out[n*K + k] = RN_fp32(w[n,k]), the value each block
 * defines ("lean" page, model table: GGUF Q4_0 / Q8_0 blocks; "oxinfer" page,
 * "How it works", quant.rs: 32 weights per scale, two nibbles per byte with
 * an f16 scale; "wgpu-llm" page, "INT8 mode": int8 with block size 64).
 * Exact for Q4_0 and Q8_0 (the product of a small integer and an fp16 scale
 * fits fp32); one IEEE rounding of c * s for LQ_I8B64 and LQ_I8B32.  out:
 * N*K fp32, 16-byte aligned. */
lq_status lq_dequant_f32(int32_t fmt, const void* W, float* out,
                         int64_t N, int64_t K, void* stream);

/* Unpacked weights rounded once to fp16 (bit patterns): out[n*K + k] =
 * RN_fp16(w[n,k]), rounded from the exact value, round to nearest even,
 * subnormals kept, overflow to inf.  This is the weight tile the prefill GEMM
 * multiplies for LQ_Q4_0 / LQ_Q8_0 (the "oxinfer" page's GPU GEMMs dequantize
 * each weight tile on chip before the dense product: "Platforms and
 * accelerators"; here in fp16 for the matrix cores).  out: N*K uint16,
 * 16-byte aligned. */
lq_status lq_dequant_f16(int32_t fmt, const void* W, uint16_t* out,
                         int64_t N, int64_t K, void* stream);

/* Load-time block quantization ("oxinfer" page, "How it works": weights are
 * block-quantized at load time; "wgpu-llm" page, "INT8 mode": symmetric int8
 * with block size 64) of a row-major N x K matrix into the packed layout.
 * src: N*K finite values of dtype sdt (LQ_F32, LQ_F16 or LQ_BF16), 16-byte
 * aligned; W: lq_packed_bytes(fmt, N, K) bytes, 16-byte aligned.  The pages
 * give no rounding rule; this one, in IEEE fp32 steps (divisions correctly
 * rounded, rint = round to nearest, ties to even), per block:
 *   LQ_Q8_0:  a = max |w|; d = fp16(a / 127); c = clamp(rint(w / d), -127, 127)
 *   LQ_Q4_0:  m = the first w of largest |w|; d = fp16(m / -8);
 *             q = clamp(rint(w / d), -8, 7) + 8  (m itself becomes code 0)
 *   LQ_I8B64, LQ_I8B32 (64- or 32-code blocks):
 *             a = max |w|; s = a / 127 (fp32);   c = clamp(rint(w / s), -127, 127)
 * A zero scale gives zero weights.  Non-finite inputs give unspecified codes.
 * lq_dequant_f32 of the result is within |d| / 2 of w per element (|d| for
 * Q4_0 codes clamped at 15). */
lq_status lq_quantize(int32_t fmt, const void* src, int32_t sdt, void* W,
                      int64_t N, int64_t K, void* stream);

/* Bytes of a GEMV split-K workspace (the same for every shape): 64-bit
 * arrival counters and fp32 partial sums.  Any contents are valid input; a
 * call leaves it reusable by the next call on the same stream. */
size_t lq_gemv_workspace_bytes(void);

/* Decode GEMV: y[n] = sum_k w[n,k] * x[k] for n < N, accumulated in fp32 with
 * the weights decoded exactly.  Decode streams every dense weight once per
 * token and is bound by memory bandwidth ("oxinfer" page, "Performance"); its
 * kernels take the quantized blocks directly ("How it works", quant.rs).
 * W: packed N x K; x: K values of dtype xdt; y: N fp32.  ws / ws_bytes: a
 * GEMV workspace (above) or NULL / 0.  Accuracy: |y - y_exact| <= 1e-4 *
 * sum_k |w x| + 1e-6 per row.  A NaN scale makes the rows it enters NaN; an
 * infinite scale makes them non-finite (see the readings in the design
 * notes: the scale multiplies each block's exact sum, so where the per-weight
 * expansion gives NaN the result may be +-inf). */
lq_status lq_gemv(int32_t fmt, const void* W, const void* x, int32_t xdt,
                  float* y, int64_t N, int64_t K, void* ws, size_t ws_bytes,
                  void* stream);

/* One independent GEMV for lq_gemv_batch (fields as in lq_gemv). */
typedef struct lq_gemv_desc {
    int32_t fmt;
    int32_t xdt;
    const void* W;
    const void* x;
    float* y;
    int64_t N;
    int64_t K;
} lq_gemv_desc;

/* Grouped launch of `count` independent GEMVs (for example every projection of
 * a decoder layer), so that small matrices share launches: a decode step
 * issues many small parallel regions whose dispatch cost matters ("oxinfer"
 * page, "How it works", pool.rs).  descs: HOST array of `count` descriptors
 * (count >= 1), read during the call only; descriptors of one format and
 * activation dtype run in one kernel launch (up to 16 per launch).  ws /
 * ws_bytes as in lq_gemv (one workspace serves the whole call).  Every
 * descriptor is validated before anything is enqueued. */
lq_status lq_gemv_batch(const lq_gemv_desc* descs, int32_t count, void* ws, size_t ws_bytes,
                        void* stream);

/* lq_gemv_batch for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same launches and results as lq_gemv_batch with a workspace, but the
 * workspace is a static array inside the library (lq_gemv_workspace_bytes()
 * bytes, 4.5 MiB, one per device, held until the process ends); nothing is
 * allocated.  That array needs no clearing, but every call on a device
 * shares it: calls that overlap in time on one device (unordered streams,
 * several threads) race and give wrong results.  Calls on one stream are
 * safe.  Every launch fits the array (K is split only within it), so no
 * shape is rejected for its size. */
lq_status lq_gemv_batch_noalloc(const lq_gemv_desc* descs, int32_t count, void* stream);

/* Multi-token GEMV, the decode step of a few tokens at once (verification of
 * drafted tokens: "oxinfer" page, "Speculative decoding", and the multi-token
 * variants of its decode kernels in "How it works"):
 *   Y[m, n] = sum_k w[n,k] * X[m,k]   for m < M, n < N,
 * every weight read once for all M tokens.  The weights are decoded exactly
 * (fp16 x exact integer code, fp32 block sums), the block scale applied in
 * fp32: for M <= 2 (LQ_Q4_0) or M <= 4 (the int8-coded formats) as lq_gemv does
 * it, each token row then being lq_gemv of that row (fp16 x) bit for bit;
 * for more tokens on the matrix cores.  W: packed N x K; X: M x K fp16
 * row-major (xdt must be LQ_F16, else LQ_ERR_UNSUPPORTED); Y: M x N fp32
 * row-major.  1 <= M <= 16, else LQ_ERR_SHAPE.  Accuracy as lq_gemv, per
 * output: |Y - Y_exact| <= 1e-4 * sum_k |w x| + 1e-6.  ws / ws_bytes: a GEMV
 * workspace or NULL / 0, as in lq_gemv. */
lq_status lq_gemv_multi(int32_t fmt, const void* W, const void* X, int32_t xdt,
                        float* Y, int64_t M, int64_t N, int64_t K, void* ws,
                        size_t ws_bytes, void* stream);

/* One independent multi-token GEMV for lq_gemv_multi_batch (fields as in
 * lq_gemv_multi; M may differ between descriptors). */
typedef struct lq_gemv_multi_desc {
    int32_t fmt;
    int32_t xdt;
    const void* W;
    const void* X;
    float* Y;
    int64_t M;
    int64_t N;
    int64_t K;
} lq_gemv_multi_desc;

/* Grouped launch of `count` independent multi-token GEMVs (for example every
 * projection of a decoder layer verifying the same drafted tokens), so that
 * small matrices share launches.  descs: HOST array of `count` descriptors
 * (count >= 1), read during the call only; all are validated before anything
 * is enqueued.  Descriptors of one format run in one kernel launch (up to 16
 * per launch), except that each M run on the lq_gemv kernel (see
 * lq_gemv_multi) takes a launch of its own.  ws / ws_bytes as in lq_gemv. */
lq_status lq_gemv_multi_batch(const lq_gemv_multi_desc* descs, int32_t count, void* ws,
                              size_t ws_bytes, void* stream);

/* Activation quantization for the integer-dot GEMV below.  The "oxinfer"
 * page quantizes each matmul's activations and takes int8 dot products of
 * them with the quantized weights ("How it works", quant.rs); it gives no
 * rounding rule, and the one here is its own Q8 rule ("How it works": 32
 * weights per scale) applied to activations.  For each token m < M and each
 * 32-element block b of its row, in fp32:
 *   s[m, b]   = max |X[m, k]| over the block / 127
 *   q[m, k]   = clamp(rint(X[m, k] / s[m, b]), -127, 127), rint rounding
 *               half to even (all codes 0 when s[m, b] = 0)
 *   sum[m, b] = sum of the block's 32 codes
 * so that |X - q s| <= s / 2 elementwise.  X: M x K, dtype xdt (LQ_F32 or
 * LQ_F16), row-major, 16-byte aligned, finite (a block holding an infinity
 * or NaN gets unspecified codes and scale).  q: M x K int8, 16-byte aligned;
 * s: M x K/32 fp32; sum: M x K/32 int32 (both 4-byte aligned; all row-major).
 * M >= 1, K a multiple of 32 (K <= 2^25), M * K / 32 <= 2^31 - 256. */
lq_status lq_quantize_act(const void* X, int32_t xdt, int64_t M, int64_t K,
                          int8_t* q, float* s, int32_t* sum, void* stream);

/* Activation-quantized decode GEMV for 1 <= M <= 16 tokens (the "oxinfer"
 * page's int8 dot-product decode kernels, "How it works", quant.rs, with their
 * multi-token variants for drafted tokens, "Speculative decoding"):
 *   Y[m, n] = sum over blocks b of (ws[n, b] * s[m, b]) * I[m, n, b],
 *   I[m, n, b] = sum over the block's 32 k of c[n, k] * q[m, k]  (exact int)
 * with c the weight's integer code (Q4_0: stored nibble - 8; Q8_0 and the
 * int8 formats: the int8 code), ws its block scale (LQ_I8B64's scale covers
 * two activation blocks), and q, s, sum as lq_quantize_act writes them (sum
 * is read for LQ_Q4_0 only, but must be valid for every format).  Every
 * weight is read once for all M tokens.  The block sums I are exact (int8
 * dot products with int32 accumulation: on the vector units for few tokens,
 * on the integer matrix cores for more); each is scaled by fl(ws * s) and
 * accumulated in fp32.  Accuracy: |Y - Y_q| <= 1e-4 * sum_b |ws s I| + 1e-6
 * per output, Y_q the exact value of the sum above.  W: packed N x K; q / s /
 * sum: M tokens of K codes, K/32 scales and K/32 sums (alignment as in
 * lq_quantize_act); Y: M x N fp32 row-major, 4-byte aligned.  ws / ws_bytes:
 * a GEMV workspace or NULL / 0, as in lq_gemv.  M outside [1, 16] is
 * LQ_ERR_SHAPE. */
lq_status lq_gemv_q8act(int32_t fmt, const void* W, const int8_t* q, const float* s,
                        const int32_t* sum, float* Y, int64_t M, int64_t N, int64_t K,
                        void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes lq_gemm needs for these arguments (0 means none): the fp32
 * partial products of K slices when the GEMM splits K across workgroups.
 * Like every buffer it is the caller's memory, borrowed for the call (the
 * "oxinfer" page's host owns GPU memory and the module only borrows it:
 * "Browser (WebGPU)", gpu_upload / gpu_matmul; "Pre-quantized checkpoints",
 * QBuf). */
size_t lq_gemm_workspace_bytes(int32_t fmt, int64_t M, int64_t N, int64_t K);

/* Prefill GEMM ("oxinfer" page, "Performance": prefill is compute bound;
 * "Platforms and accelerators": weights dequantized on chip for a dense tile
 * product), every format, fp16 X (xdt must be LQ_F16, else
 * LQ_ERR_UNSUPPORTED), products and sums in fp32 on the matrix cores:
 *   LQ_Q4_0, LQ_Q8_0:  Y[m,n] = sum_k RN_fp16(w[n,k]) * X[m,k]
 *                      (the fp16 tile of lq_dequant_f16);
 *   LQ_I8B64, LQ_I8B32: Y[m,n] = sum_blocks s * sum_k c[n,k] * X[m,k]
 *                      (codes exact, fp32 scale applied to block sums).
 * W: packed N x K; X: M x K fp16 row-major; Y: M x N fp32 row-major.
 * ws / ws_bytes: workspace of at least lq_gemm_workspace_bytes() bytes (may
 * be NULL when that is 0).  Accuracy: |Y - Y_exact| <= 2e-3 * sum_k |w x| +
 * 1e-5 per element. */
lq_status lq_gemm(int32_t fmt, const void* W, const void* X, int32_t xdt,
                  float* Y, int64_t M, int64_t N, int64_t K,
                  void* ws, size_t ws_bytes, void* stream);

/* One weight matrix of lq_gemm_batch: W packed N x K, Y M x N fp32. */
typedef struct lq_gemm_desc {
    const void* W;
    float* Y;
    int64_t N;
} lq_gemm_desc;

/* Most matrices one lq_gemm_batch call takes. */
#define LQ_GEMM_MAX_GROUP 4

/* lq_gemm over `count` weight matrices (1 <= count <= LQ_GEMM_MAX_GROUP) of
 * one format that share X, M and K, e.g. the gate and up projections of one
 * FFN over the same prompt chunk: for each descriptor, Y = X W^T as lq_gemm
 * computes it (the same fp16 weight tile and products, with the same
 * accuracy; the same bits whenever lq_gemm needs no workspace for that matrix
 * alone, i.e. does not split its K).  All of them run in one kernel launch,
 * so their output tiles fill the GPU together.  descs: HOST array, read
 * during the call only; everything is validated before anything is enqueued.
 * ws / ws_bytes: a workspace of the largest lq_gemm_workspace_bytes() over
 * the descriptors suffices (a call with count > 1 needs none). */
lq_status lq_gemm_batch(int32_t fmt, const void* X, int32_t xdt, int64_t M, int64_t K,
                        const lq_gemm_desc* descs, int32_t count,
                        void* ws, size_t ws_bytes, void* stream);

/* Route by token count, after the "oxinfer" page's rule that the dense-tile
 * GPU matmul takes only prompt-sized work ("Platforms and accelerators": t >=
 * 16 tokens): M == 1 runs lq_gemv on X (fp32 or fp16); 2 <= M <= 16 with fp16
 * X runs lq_gemv_multi (its matrix-core fragment holds 16 tokens, and it is
 * faster than the tile GEMM there); everything else runs lq_gemm.  Arguments
 * as in lq_gemm; the GEMV paths use ws as their workspace when ws_bytes >=
 * lq_gemv_workspace_bytes(), else none. */
lq_status lq_matmul(int32_t fmt, const void* W, const void* X, int32_t xdt,
                    float* Y, int64_t M, int64_t N, int64_t K,
                    void* ws, size_t ws_bytes, void* stream);

/* Name of a status code ("LQ_OK", ...). */
const char* lq_status_str(int32_t status);

/* Message of the calling thread's last failed call ("" if none). */
const char* lq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LQ_H */
