// Internal declarations shared by the liblq translation units (host side of
// the launches plus the argument blocks the kernels receive).  Not installed.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace lq {

enum Fmt : int { kQ4_0 = 0, kQ8_0 = 1, kI8B64 = 2, kI8B32 = 3 };
enum XType : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

// ------------------------------------------------------ packed layout ----
// Rows are grouped in tiles of 64.  A "unit" is one scale block of a row
// (32 weights for Q4_0 / Q8_0, 64 for int8 block-64) and its codes are cut
// into 16-byte parts (1, 2 or 4).  Inside a tile the codes are stored
// unit-major, then part, then row: the 64 rows' copies of one part of one
// unit are one contiguous 1 KB run, so one wave whose lane r owns row r of
// the tile reads it with a single coalesced 16-byte-per-lane load.  The last
// tile of a matrix may hold fewer than 64 rows (nr); its runs are nr * 16
// bytes and nothing is padded.  The scale plane is laid out the same way with
// one 2- or 4-byte scale in place of a 16-byte part.
constexpr int kTileRows = 64;
__host__ __device__ constexpr int unit_elems(int fmt) { return fmt == kI8B64 ? 64 : 32; }
__host__ __device__ constexpr int unit_parts(int fmt) { return fmt == kQ4_0 ? 1 : (fmt == kI8B64 ? 4 : 2); }
__host__ __device__ constexpr int unit_bytes(int fmt) { return 16 * unit_parts(fmt); }
// Order of the loads of one GEMV batch: all the units' scale loads before
// their code loads for formats whose unit has several 16-byte code parts
// (Q8_0 decoder layer 13.0 -> 12.9 us, the layer at 2 / 4 / 16 tokens 3 %
// faster); for Q4_0 each unit's scale load right after its code load (the
// LM head took 14.8 us with the scales first and 15.4 us with all codes,
// then all scales, against 14.4 us).
__host__ __device__ constexpr bool scales_first(int fmt) { return unit_parts(fmt) > 1; }
// fp32 scales (int8 block-64 and block-32): the codes stay exact and the
// scale multiplies fp32 sums; fp16 scales (Q4_0, Q8_0).
__host__ __device__ constexpr bool fp32_scale(int fmt) { return fmt == kI8B64 || fmt == kI8B32; }
__host__ __device__ constexpr int scale_bytes(int fmt) { return fp32_scale(fmt) ? 4 : 2; }

inline size_t code_plane_bytes(int fmt, int64_t N, int64_t K) {
    return fmt == kQ4_0 ? size_t(N) * size_t(K) / 2 : size_t(N) * size_t(K);
}
inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
inline size_t scale_plane_bytes(int fmt, int64_t N, int64_t K) {
    return size_t(N) * size_t(K / unit_elems(fmt)) * size_t(scale_bytes(fmt));
}

// Position of (row, unit) in the tiled layout: `code` is the byte offset of
// part 0 (part p adds p * nr * 16), `scale` the index of the unit's scale.
struct TiledPos {
    size_t code;
    size_t scale;
    uint32_t part_stride;   // nr * 16
};
__host__ __device__ inline TiledPos tiled_pos(int fmt, int64_t N, int64_t nu, int64_t row, int64_t u) {
    const int64_t tile = row / kTileRows;
    const int64_t r = row - tile * kTileRows;
    const int64_t rest = N - tile * kTileRows;
    const int64_t nr = rest < kTileRows ? rest : kTileRows;
    const int64_t first = tile * kTileRows * nu;   // units stored before this tile
    TiledPos p;
    p.code = size_t(first + u * nr) * size_t(unit_bytes(fmt)) + size_t(r) * 16;
    p.scale = size_t(first + u * nr + r);
    p.part_stride = uint32_t(nr * 16);
    return p;
}

// ---------------------------------------------------------------- GEMV ----
constexpr int kMaxBatch = 16;       // descriptors per grouped launch
constexpr int kGemvThreads = 256;   // 4 waves: one tile, K split four ways
// Waves per workgroup of a GEMV launch whose matrices all split K across at
// least this many workgroups of 4 waves: the split then moves inside one
// workgroup of 16 waves.
#ifndef LQ_GEMV_WIDE_FROM
#define LQ_GEMV_WIDE_FROM 4
#endif
// Split-K workspace of the GEMV calls (the caller's memory, lq_gemv_workspace_bytes):
// one 64-bit arrival counter per tile of the split matrices, then the
// partial sums of their K slices.  A launch splits K only if both fit.
constexpr int64_t kGemvCounters = int64_t(1) << 16;     // 512 KiB
constexpr int64_t kGemvPartFloats = int64_t(1) << 20;   // 4 MiB
constexpr size_t kGemvWorkspaceBytes = size_t(kGemvCounters) * 8 + size_t(kGemvPartFloats) * 4;
// Most K slices of one tile (the arrival count is a 16-bit field).
constexpr int64_t kMaxSlices = 4096;

// Matrix of workgroup `bid` in a grouped launch.  wg0[i] is the first
// workgroup of matrix i, INT32_MAX past the last matrix; the matrix is the
// number of entries after the first that are not after bid.  The table
// arrives in one scalar load and the count is two scalar instructions per
// entry (compare, add the carry).  A loop over the descriptors themselves
// made one dependent scalar load per matrix before a wave's first weight
// load (0.6 us of the 13.8 us Q8_0 decoder-layer launch), and every scalar
// instruction before that load counts: the CU's one scalar unit serves all
// its waves (64 more of them in the prologue cost that launch 0.25 us).
template <int NB>
__device__ inline int find_matrix(const int32_t (&wg0)[NB], int bid) {
    int di = 0;
    if constexpr (NB == 16) {
        // One block, so that no filler instructions separate the pairs.
#define LQ_CMP_ADD(i) "s_cmp_ge_i32 %1, %" #i "\n\ts_addc_u32 %0, %0, 0\n\t"
        asm(LQ_CMP_ADD(2) LQ_CMP_ADD(3) LQ_CMP_ADD(4) LQ_CMP_ADD(5) LQ_CMP_ADD(6) LQ_CMP_ADD(7) LQ_CMP_ADD(8)
                LQ_CMP_ADD(9) LQ_CMP_ADD(10) LQ_CMP_ADD(11) LQ_CMP_ADD(12) LQ_CMP_ADD(13) LQ_CMP_ADD(14)
                    LQ_CMP_ADD(15) LQ_CMP_ADD(16)
            : "+s"(di)
            : "s"(bid), "s"(wg0[1]), "s"(wg0[2]), "s"(wg0[3]), "s"(wg0[4]), "s"(wg0[5]), "s"(wg0[6]),
              "s"(wg0[7]), "s"(wg0[8]), "s"(wg0[9]), "s"(wg0[10]), "s"(wg0[11]), "s"(wg0[12]), "s"(wg0[13]),
              "s"(wg0[14]), "s"(wg0[15])
            : "scc");
#undef LQ_CMP_ADD
    } else {
#pragma unroll
        for (int i = 1; i < NB; ++i)
            asm("s_cmp_ge_i32 %1, %2\n\ts_addc_u32 %0, %0, 0" : "+s"(di) : "s"(bid), "s"(wg0[i]) : "scc");
    }
    return di;
}
template <int NB, class Desc>
inline void fill_wg0_table(int32_t (&t)[NB], const Desc (&d)[NB], int count) {
    for (int i = 0; i < NB; ++i) t[i] = i < count ? d[i].wg0 : INT32_MAX;
}

// Units [sa, sb) of slice `slice` of S over nu units: floor(nu * slice / S)
// and floor(nu * (slice + 1) / S), in 32-bit arithmetic.  With nu = q S + r,
// floor(nu s / S) = q s + floor(r s / S), and r s < S * S fits in 32 bits.
static_assert(kMaxSlices < 65536, "32-bit slice bounds");
__device__ inline void slice_units(int nu, int S, int slice, int& sa, int& sb) {
    const uint32_t s = uint32_t(S), q = uint32_t(nu) / s, r = uint32_t(nu) - q * s;
    sa = int(q * uint32_t(slice) + r * uint32_t(slice) / s);
    sb = int(q * uint32_t(slice + 1) + r * uint32_t(slice + 1) / s);
}
// Workgroups a launch aims for per CU before it splits K across workgroups,
// and the fewest units a wave keeps when K is split.
#ifndef LQ_GEMV_WGS_PER_CU
#define LQ_GEMV_WGS_PER_CU 8
#endif
// Most units whose loads one wave issues before computing them (per
// format).  A launch whose waves have at most u units runs them in
// ceil(u / cap) batches of equal size (the kernel is instantiated for every
// batch size up to the cap).
#ifndef LQ_GEMV_UNR_Q4
#define LQ_GEMV_UNR_Q4 8
#endif
#ifndef LQ_GEMV_UNR_Q8
#define LQ_GEMV_UNR_Q8 4
#endif
// The same for Q8_0 and int8 block-32 launches of three or more tokens
// (their activations take the registers).
#ifndef LQ_GEMV_UNR_Q8_TOKENS
#define LQ_GEMV_UNR_Q8_TOKENS 2
#endif
#ifndef LQ_GEMV_UNR_I8
#define LQ_GEMV_UNR_I8 1
#endif
// Most units a sub-tile GEMV wave (launch_gemv_sub) loads before computing
// them, one token.
#ifndef LQ_GEMV_SUB_UNR
#define LQ_GEMV_SUB_UNR 4
#endif
// Fewest units a wave keeps when K is split, per format (a unit is 1, 2 or
// 4 KB of codes per wave for Q4_0, Q8_0, int8 block-64).
#ifndef LQ_GEMV_MIN_UNITS_Q4
#define LQ_GEMV_MIN_UNITS_Q4 8
#endif
#ifndef LQ_GEMV_MIN_UNITS_Q8
#define LQ_GEMV_MIN_UNITS_Q8 4
#endif
#ifndef LQ_GEMV_MIN_UNITS_I8
#define LQ_GEMV_MIN_UNITS_I8 2
#endif
// Launches of formats with several code parts per unit whose tiles, split
// by rows into unit_parts(fmt) workgroups each, are no more than the
// device's CUs split tiles that way (launch_gemv_sub), for any token count,
// when no matrix has more than this many units per row (16 waves then get at most 8
// units each); longer rows keep the K split across workgroups.
#ifndef LQ_GEMV_SUB_MAX_UNITS
#define LQ_GEMV_SUB_MAX_UNITS 128
#endif
inline int gemv_min_units(int fmt) {
    return fmt == kQ4_0 ? LQ_GEMV_MIN_UNITS_Q4 : (fmt == kI8B64 ? LQ_GEMV_MIN_UNITS_I8 : LQ_GEMV_MIN_UNITS_Q8);
}
// The same for the multi-token GEMV (4-wave workgroups), whose split K also
// moves M tokens of partial sums per row through the workspace, so it pays
// to split less: in grouped launches the K = 2048 matrices of a layer are
// best left unsplit and a long-K matrix split a few ways.  Measured on
// grouped layers (M = 5 / 8 / 12 / 16): the Q8_0 layer from 21.3 / 22.2 /
// 24.9 / 28.0 us (8 units) to 17.8 / 17.9 / 18.9 / 19.6 (16; 12 and 24 were
// slower), the Q4_0 2048 / 11008 FFN from 21.6 / 22.6 / 25.4 / 28.3 (8) to
// 16.9 / 17.3 / 18.1 / 19.0 (16; 32 and 64 slower), the int8 block-64 layer
// from 22.5 / 24.3 / 27.8 / 23.0 (2 units of 64 weights) to 17.0 / 17.6 (4,
// M <= 8) and 18.9 / 20.0 (8, M > 8).
#ifndef LQ_MULTI_MIN_UNITS_Q4
#define LQ_MULTI_MIN_UNITS_Q4 16
#endif
#ifndef LQ_MULTI_MIN_UNITS
#define LQ_MULTI_MIN_UNITS 16
#endif
#ifndef LQ_MULTI_MIN_UNITS_I8
#define LQ_MULTI_MIN_UNITS_I8 4
#endif
#ifndef LQ_MULTI_MIN_UNITS_I8_MANY
#define LQ_MULTI_MIN_UNITS_I8_MANY 8
#endif
inline int multi_min_units(int fmt, int64_t M) {
    if (fmt == kI8B64) return M <= 8 ? LQ_MULTI_MIN_UNITS_I8 : LQ_MULTI_MIN_UNITS_I8_MANY;
    return fmt == kQ4_0 ? LQ_MULTI_MIN_UNITS_Q4 : LQ_MULTI_MIN_UNITS;
}

struct GemvDesc {
    const uint8_t* codes;   // code plane (tiled)
    const uint8_t* scales;  // scale plane (tiled)
    const void* x;          // activations (fp32 or fp16): MT rows of K values
    float* y;               // MT rows of N outputs
    float* part;            // split-K partials: S slices x MT tokens x tiles * 64 floats (S > 1 only)
    uint64_t* cnt;          // one arrival counter per tile (S > 1 only)
    int32_t N;              // rows
    int32_t nu;             // units per row (K / unit_elems)
    int32_t tiles;          // ceil(N / 64)
    int32_t S;              // K slices (workgroups per tile)
    int32_t wg0;            // first workgroup of this matrix in the launch
    uint32_t tile_bytes;    // code bytes of one 64-row tile (64 * nu * unit_bytes)
};

struct GemvArgs {
    int32_t wg0[kMaxBatch]; // d[i].wg0, INT32_MAX past count (find_matrix)
    GemvDesc d[kMaxBatch];
    uint64_t tag;           // this launch's split-K tag (splitk_arrive)
    int32_t count;
    int32_t total_wgs;
};

// A split-K tag for a new launch: nonzero, 48 bits, never repeated in the
// process (a captured graph replays the tag it was captured with).
uint64_t next_splitk_tag();

// Most tokens one GEMV launch takes (MT > 1 only with fp16 activations).
// Every weight is decoded once for all tokens, and each token adds one fp16
// dot product per weight pair: Q4_0 (the costliest decode per byte) stays
// under the weight stream's time up to two tokens, Q8_0 and int8 block-64
// up to four.
__host__ __device__ constexpr int gemv_max_tokens(int fmt) { return fmt == kQ4_0 ? 2 : 4; }
// mt: tokens of the launch, 1 .. gemv_max_tokens(fmt).
hipError_t launch_gemv(int fmt, int xdt, int waves, int mt, const GemvArgs& args, hipStream_t stream);
// Q8_0 / int8 block-64, mt tokens (as launch_gemv), K unsplit: each 64-row
// tile is split by rows across unit_parts(fmt) workgroups of 16 waves
// (args.total_wgs counts those workgroups, d[i].wg0 the first of matrix i,
// d[i].S must be 1).
hipError_t launch_gemv_sub(int fmt, int xdt, int mt, const GemvArgs& args, hipStream_t stream);

// ------------------------------------------------- multi-token GEMV ----
constexpr int kMultiMaxTokens = 16;   // tokens of one MFMA fragment
// Units whose loads one wave issues before computing them (per format).
#ifndef LQ_MULTI_UNR_Q4
#define LQ_MULTI_UNR_Q4 4
#endif
#ifndef LQ_MULTI_UNR_Q8
#define LQ_MULTI_UNR_Q8 2
#endif
#ifndef LQ_MULTI_UNR_I8
#define LQ_MULTI_UNR_I8 2
#endif
// Q4_0 launches whose waves all have more than LQ_MULTI_UNR_Q4 and at most
// this many units (K = 896 on one slice: 7) load them in one batch instead of
// two.  Longer loops keep the smaller batch, which needs fewer registers.
#ifndef LQ_MULTI_UNR_Q4_ONE
#define LQ_MULTI_UNR_Q4_ONE 7
#endif

struct MultiDesc {
    const uint8_t* codes;   // code plane (tiled)
    const uint8_t* scales;  // scale plane (tiled)
    const _Float16* x;      // M x K activations, row-major
    float* y;               // M x N outputs, row-major
    float* part;            // split-K partials: S slices x M tokens x tiles * 64 floats (S > 1 only)
    uint64_t* cnt;          // one arrival counter per tile (S > 1 only)
    int32_t N;              // rows (and the row pitch of y)
    int32_t K;              // reduction length (and the row pitch of x)
    int32_t nu;             // units per row
    int32_t tiles;          // ceil(N / 64)
    int32_t S;              // K slices (workgroups per tile)
    int32_t M;              // tokens, 1 .. kMultiMaxTokens
    int32_t vec_y;          // y rows are 16-byte aligned: full tiles store float4
    int32_t wg0;            // first workgroup of this matrix in the launch
};

struct MultiArgs {
    int32_t wg0[kMaxBatch]; // d[i].wg0, INT32_MAX past count (find_matrix)
    MultiDesc d[kMaxBatch];
    uint64_t tag;           // this launch's split-K tag (splitk_arrive)
    int32_t count;
    int32_t total_wgs;
};

hipError_t launch_gemv_multi(int fmt, const MultiArgs& a, hipStream_t stream);

// ------------------------------------- activation-quantized GEMV ----
// Activations quantized per 32-element block to int8 codes q (M x K), fp32
// scales s and code sums (M x K / 32 each); Y = sum over blocks of
// (w_scale * s) * (integer block dot product).
constexpr int kQ8ActMaxTokens = 16;
// Token counts from which the integer-dot GEMV runs on the matrix cores
// (fewer run on the vector dot-product kernel).  Measured kernel times, LM
// head 151936x896 Q4_0 at M = 6 / 8 / 16: 20.7 / 23.7 / 40 us (vector) and
// 20.7 / 21.5 / 24.7 us (matrix cores); the int8 formats' vector kernel is
// faster up to M = 8 on every shape measured (Q8_0 8192x2048 at M = 8:
// 8.1 vs 11.0 us) and the matrix cores at M = 16 are even or ahead (Q8_0
// 2048x8192: 22.1 vs 16.6 us).
#ifndef LQ_Q8ACT_MFMA_FROM_Q4
#define LQ_Q8ACT_MFMA_FROM_Q4 7
#endif
#ifndef LQ_Q8ACT_MFMA_FROM_I8
#define LQ_Q8ACT_MFMA_FROM_I8 16
#endif
__host__ __device__ constexpr int q8act_mfma_from(int fmt) {
    return fmt == kQ4_0 ? LQ_Q8ACT_MFMA_FROM_Q4 : LQ_Q8ACT_MFMA_FROM_I8;
}

struct Q8ActArgs {
    const uint8_t* codes;   // code plane (tiled)
    const uint8_t* scales;  // scale plane (tiled)
    const int8_t* q;        // M x K activation codes, row-major
    const float* s;         // M x K/32 activation scales
    const int32_t* sum;     // M x K/32 code sums (Q4_0's offset of 8)
    float* y;               // M x N outputs, row-major
    float* part;            // split-K partials: S slices x M tokens x tiles * 64 floats (S > 1 only)
    uint64_t* cnt;          // one arrival counter per tile (S > 1 only)
    uint64_t tag;           // this launch's split-K tag (splitk_arrive)
    int32_t N;              // rows
    int32_t nu;             // units per row
    int32_t tiles;          // ceil(N / 64)
    int32_t S;              // K slices (workgroups per tile)
    int32_t M;              // tokens, 1 .. kQ8ActMaxTokens
    int32_t pad;
};
hipError_t launch_quantize_act(int xdt, const void* X, int64_t M, int64_t K, int8_t* q, float* s, int32_t* sum,
                               hipStream_t stream);
// waves: 4 or 16 per workgroup (the units of one K slice are split among them).
hipError_t launch_gemv_q8act(int fmt, const Q8ActArgs& a, int waves, hipStream_t stream);
// The same product on the integer matrix cores (4 waves per workgroup, one
// 64-row tile per K slice; partials of M tokens per slice as above).
hipError_t launch_gemv_q8act_mfma(int fmt, const Q8ActArgs& a, hipStream_t stream);

// ------------------------------------------------------- conversions ----
hipError_t launch_repack_gguf(int fmt, const void* src, void* dst, int64_t N, int64_t K,
                              hipStream_t stream);
hipError_t launch_pack_planes(int fmt, const void* codes, const void* scales, void* dst, int64_t N,
                              int64_t K, hipStream_t stream);
hipError_t launch_quantize(int fmt, int sdt, const void* src, void* dst, int64_t N, int64_t K,
                           hipStream_t stream);
hipError_t launch_dequant(int fmt, bool to_f16, const void* W, void* out, int64_t N,
                          int64_t K, hipStream_t stream);

// ---------------------------------------------------------------- GEMM ----
// Matrices one tile GEMM launch takes (they share X, M and K).
constexpr int kMaxGemmGroup = 4;
// Split-K workspace of a single-matrix launch (0: none).  Launches of
// several matrices never split K.
size_t gemm_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K);
// Weights decoded to fp16 tiles in LDS: Q4_0 and Q8_0 as RN_fp16(q d),
// int8 block-64 as exact codes with the fp32 scale applied to block sums.
hipError_t launch_gemm_tile(int fmt, const void* const* W, float* const* Y, const int64_t* N, int count,
                            const void* X, int64_t M, int64_t K, void* ws, int num_cus,
                            hipStream_t stream);
// Y = sum of S partial M x N slices (slice order), for split-K GEMMs.
hipError_t launch_splitk_reduce(const float* P, float* Y, size_t mn, int S, hipStream_t stream);

}  // namespace lq
