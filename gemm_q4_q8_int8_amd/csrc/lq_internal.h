// Internal declarations shared by the liblq translation units (host side of
// the launches plus the argument blocks the kernels receive).  Not installed.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace lq {

enum Fmt : int { kQ4_0 = 0, kQ8_0 = 1, kI8B64 = 2 };
enum XType : int { kF32 = 0, kF16 = 1 };

// Code bytes per 32-weight unit and scale bytes per scale.
constexpr int unit_code_bytes(int fmt) { return fmt == kQ4_0 ? 16 : 32; }

// Packed-layout geometry (the layout documented in lq.h).
inline size_t code_plane_bytes(int fmt, int64_t N, int64_t K) {
    return fmt == kQ4_0 ? size_t(N) * size_t(K) / 2 : size_t(N) * size_t(K);
}
inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
inline size_t scale_plane_bytes(int fmt, int64_t N, int64_t K) {
    return fmt == kI8B64 ? size_t(N) * size_t(K / 64) * 4 : size_t(N) * size_t(K / 32) * 2;
}

// ---------------------------------------------------------------- GEMV ----
constexpr int kMaxBatch = 16;       // descriptors per grouped launch
constexpr int kGemvThreads = 256;
// Rows per team per step: 8 for Q4_0 (16-byte units), 4 for the 32-byte int8
// units, so two steps of code registers fit without spilling.
#ifndef LQ_GEMV_RPI_Q4
#define LQ_GEMV_RPI_Q4 8
#endif
#ifndef LQ_GEMV_RPI_I8
#define LQ_GEMV_RPI_I8 4
#endif
// Steps of weight loads kept in flight per wave (register ring depth - 1).
#ifndef LQ_GEMV_NBUF
#define LQ_GEMV_NBUF 2
#endif
// Resident GEMV workgroups per CU (persistent grid size = CUs x this).
#ifndef LQ_GEMV_WGS_PER_CU
#define LQ_GEMV_WGS_PER_CU 2
#endif
constexpr int gemv_rpi(int fmt) { return fmt == kQ4_0 ? LQ_GEMV_RPI_Q4 : LQ_GEMV_RPI_I8; }
constexpr int kGemvXLdsFloats = 16384;   // LDS budget (floats) for a launch's activations

struct GemvDesc {
    const uint8_t* codes;   // code plane
    const void* scales;     // scale plane (fp16 or fp32)
    const void* x;          // activations in global memory (fp32 or fp16)
    float* y;               // output rows
    int32_t N;              // rows
    int32_t nu;             // 32-weight units per row (K / 32)
    int32_t xdt;            // kF32 / kF16
    int32_t nchunks;        // chunks of TP units per row
    int32_t iters;          // row iterations (rows_per_iter rows each)
    int32_t iter0;          // first row iteration of this matrix in the launch
    int32_t x_off;          // LDS offset (floats) of its staged activations
    int32_t pad;
};

// One activation vector staged in LDS at the start of a launch.
struct GemvXSrc {
    const void* x;
    int32_t K;
    int32_t xdt;
    int32_t lds_off;        // floats, a multiple of 32
    int32_t pad;
};

struct GemvBatchArgs {
    GemvDesc d[kMaxBatch];
    GemvXSrc xs[kMaxBatch];
    int32_t nx;             // activation vectors to stage
    int32_t total_iters;
    int32_t count;
    int32_t pad;
};

// A team of `tp` lanes owns one row at a time; lane t of a team handles unit
// t of each chunk of tp units.
struct GemvConfig {
    int tp;
    int rpi;
    int rows_per_iter;   // rows one workgroup covers per step
    bool x_global;       // activations read from global memory (K too long for LDS)
};

GemvConfig gemv_config(int fmt, int nu);
hipError_t launch_gemv(int fmt, const GemvConfig& cfg, const GemvBatchArgs& args,
                       int grid, size_t lds_bytes, hipStream_t stream);

// ------------------------------------------------------- conversions ----
hipError_t launch_repack_gguf(int fmt, const void* src, void* dst, int64_t N, int64_t K,
                              hipStream_t stream);
hipError_t launch_dequant(int fmt, bool to_f16, const void* W, void* out, int64_t N,
                          int64_t K, hipStream_t stream);

// ---------------------------------------------------------------- GEMM ----
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_q4_0(const void* W, const void* X, float* Y, int64_t M, int64_t N,
                            int64_t K, void* ws, size_t ws_bytes, int num_cus,
                            hipStream_t stream);

}  // namespace lq
