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
constexpr int kMaxBatch = 16;     // descriptors per grouped launch
constexpr int kGemvThreads = 256;

struct GemvDesc {
    const uint8_t* codes;   // code plane
    const void* scales;     // scale plane (fp16 or fp32)
    const void* x;          // activations (fp32 or fp16)
    float* y;               // output rows
    int32_t N;              // rows
    int32_t nu;             // 32-weight units per row (K / 32)
    int32_t xdt;            // kF32 / kF16
    int32_t iters;          // row iterations of this descriptor
};

struct GemvBatchArgs {
    GemvDesc d[kMaxBatch];
    int32_t prefix[kMaxBatch + 1];   // prefix sums of iters
    int32_t count;
};

// A team of `tp` lanes owns one row at a time; lane t of a team holds the
// activations of units t, t + tp, ... (`upl` of them) in registers.
struct GemvConfig {
    int tp;
    int upl;
    int rows_per_iter;   // rows one workgroup covers per iteration
};

GemvConfig gemv_config(int nu);
hipError_t launch_gemv(int fmt, const GemvConfig& cfg, const GemvBatchArgs& args,
                       int grid, hipStream_t stream);

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
