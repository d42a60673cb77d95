// Layout conversion and exact unpacking.
//
//   repack_gguf: GGUF array-of-blocks (fp16 scale then codes, 18 or 34 bytes
//   per block, only 2-byte aligned) -> the tiled packed layout (64-row tiles,
//   unit-major, each 16-byte code part of a unit stored for the tile's rows
//   side by side).  Pure byte moves.
//
//   pack_planes: row-major code and scale planes -> the same tiled layout.
//
//   dequant: the unpacked-weight contract.  fp32 output is RN_fp32(w): exact
//   for Q4_0 / Q8_0 (small integer times an fp16 scale always fits fp32) and a
//   single IEEE multiply c * s for int8 block-64.  fp16 output is RN_fp16(w):
//   one fp16 multiply of the exact fp16 code by the fp16 scale for Q4_0 /
//   Q8_0; for int8 block-64 the exact product c * s needs up to 31 significant
//   bits, so it is rounded to fp16 in integer arithmetic (one rounding, round
//   to nearest even, gradual underflow) rather than through fp32.
//
//   quantize: fp32 / fp16 / bf16 row-major weights -> the packed layout
//   (load-time block quantization; the rule is stated at quantize_kernel).
//
// One thread handles one block (repack, pack, quantize) or 32 weights (dequant).  These kernels run once per weight
// upload or inside tests; they are not on the timed decode path.
#include "lq_internal.h"

namespace lq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

template <int FMT>
__global__ __launch_bounds__(kThreads) void repack_kernel(const uint16_t* __restrict__ src,
                                                          uint8_t* __restrict__ dst, int64_t N,
                                                          int64_t nu, size_t scale_off) {
    constexpr int HW = FMT == kQ4_0 ? 9 : 17;   // 16-bit words per GGUF block
    constexpr int CV = unit_parts(FMT);         // 16-byte code parts per block
    const int64_t b = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (b >= N * nu) return;
    const int64_t row = b / nu;
    const TiledPos pos = tiled_pos(FMT, N, nu, row, b - row * nu);
    const uint16_t* s = src + b * HW;
    reinterpret_cast<uint16_t*>(dst + scale_off)[pos.scale] = s[0];
#pragma unroll
    for (int v = 0; v < CV; ++v) {
        u32x4 t;
        t.x = uint32_t(s[1 + 8 * v + 0]) | (uint32_t(s[1 + 8 * v + 1]) << 16);
        t.y = uint32_t(s[1 + 8 * v + 2]) | (uint32_t(s[1 + 8 * v + 3]) << 16);
        t.z = uint32_t(s[1 + 8 * v + 4]) | (uint32_t(s[1 + 8 * v + 5]) << 16);
        t.w = uint32_t(s[1 + 8 * v + 6]) | (uint32_t(s[1 + 8 * v + 7]) << 16);
        *reinterpret_cast<u32x4*>(dst + pos.code + size_t(v) * pos.part_stride) = t;
    }
}

// Row-major code and scale planes -> tiled layout: one thread per unit.
template <int FMT>
__global__ __launch_bounds__(kThreads) void pack_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales,
                                                        uint8_t* __restrict__ dst, int64_t N,
                                                        int64_t nu, size_t scale_off) {
    constexpr int CV = unit_parts(FMT);
    constexpr int SB = scale_bytes(FMT);
    const int64_t g = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (g >= N * nu) return;
    const int64_t row = g / nu;
    const TiledPos pos = tiled_pos(FMT, N, nu, row, g - row * nu);
    const u32x4* src = reinterpret_cast<const u32x4*>(codes) + g * CV;
#pragma unroll
    for (int v = 0; v < CV; ++v)
        *reinterpret_cast<u32x4*>(dst + pos.code + size_t(v) * pos.part_stride) = src[v];
    if constexpr (SB == 2)
        reinterpret_cast<uint16_t*>(dst + scale_off)[pos.scale] = reinterpret_cast<const uint16_t*>(scales)[g];
    else
        reinterpret_cast<uint32_t*>(dst + scale_off)[pos.scale] = reinterpret_cast<const uint32_t*>(scales)[g];
}

// RN_fp16(c * s) for an int8 code c and an fp32 scale s, from the exact
// integer product of c and the significand of s.
__device__ uint16_t rn16_code_times_f32(int c, float s) {
    const uint32_t sb = __float_as_uint(s);
    const uint32_t sign = ((sb >> 31) ^ (c < 0 ? 1u : 0u)) & 1u;
    const uint32_t se = (sb >> 23) & 0xFFu;
    const uint32_t sm = sb & 0x7FFFFFu;
    if (se == 0xFFu) {  // inf or NaN scale: no rounding question
        const _Float16 h = (_Float16)(float(c) * s);
        return __builtin_bit_cast(uint16_t, h);
    }
    const uint32_t ac = uint32_t(c < 0 ? -c : c);
    if (ac == 0 || (se == 0 && sm == 0)) return uint16_t(sign << 15);
    const uint64_t A = uint64_t(ac) * uint64_t(se ? (sm | 0x800000u) : sm);  // < 2^31
    const int B = se ? int(se) - 150 : -149;                                  // |c s| = A 2^B
    const int p = 63 - __builtin_clzll(A);
    int E = p + B;                                                            // binade of |c s|
    const int qe = E >= -14 ? E - 10 : -24;                                   // fp16 quantum
    const int shift = qe - B;
    uint64_t m;
    if (shift <= 0) {
        m = A << (-shift);
    } else if (shift >= 40) {
        m = 0;  // A < 2^31 is below half a quantum
    } else {
        m = A >> shift;
        const uint64_t rem = A & ((uint64_t(1) << shift) - 1);
        const uint64_t half = uint64_t(1) << (shift - 1);
        if (rem > half || (rem == half && (m & 1))) ++m;
    }
    if (E >= -14) {
        if (m == 2048) { m = 1024; ++E; }
        if (E > 15) return uint16_t((sign << 15) | 0x7C00u);
        return uint16_t((sign << 15) | (uint32_t(E + 15) << 10) | uint32_t(m - 1024));
    }
    return uint16_t((sign << 15) | uint32_t(m));  // subnormal; m == 1024 is the smallest normal
}

template <int FMT, bool F16>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t* __restrict__ W,
                                                           void* __restrict__ out, int64_t N,
                                                           int nh, size_t scale_off) {
    // One thread per 32 weights: row `row`, 32-element group h of nh.
    const int64_t g = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (g >= N * nh) return;
    const int64_t row = g / nh;
    const int u = int(g % nh);                      // 32-element group
    const int64_t K = int64_t(nh) * 32;
    constexpr int GPU_ = unit_elems(FMT) / 32;      // groups per unit
    const int64_t nu = nh / GPU_;
    const TiledPos pos = tiled_pos(FMT, N, nu, row, u / GPU_);
    const int part0 = (u % GPU_) * 2;               // int8: two 16-byte parts per group
    int code[32];
    if (FMT == kQ4_0) {
        const u32x4 c = *reinterpret_cast<const u32x4*>(W + pos.code);
        const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t byte = (w[j / 4] >> (8 * (j % 4))) & 0xFFu;
            code[j] = int(byte & 0xFu) - 8;        // element j: low nibble
            code[j + 16] = int(byte >> 4) - 8;     // element j + 16: high nibble
        }
    } else {
        const u32x4 c0 = *reinterpret_cast<const u32x4*>(W + pos.code + size_t(part0) * pos.part_stride);
        const u32x4 c1 = *reinterpret_cast<const u32x4*>(W + pos.code + size_t(part0 + 1) * pos.part_stride);
        const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
        for (int j = 0; j < 32; ++j) code[j] = int(int8_t((w[j / 4] >> (8 * (j % 4))) & 0xFFu));
    }
    if (!F16) {
        float s;
        if (fp32_scale(FMT)) s = reinterpret_cast<const float*>(W + scale_off)[pos.scale];
        else s = float(reinterpret_cast<const _Float16*>(W + scale_off)[pos.scale]);
        f32x4* o = reinterpret_cast<f32x4*>(static_cast<float*>(out) + row * K + int64_t(u) * 32);
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            f32x4 t;
            t.x = float(code[4 * v + 0]) * s;
            t.y = float(code[4 * v + 1]) * s;
            t.z = float(code[4 * v + 2]) * s;
            t.w = float(code[4 * v + 3]) * s;
            o[v] = t;
        }
    } else {
        uint16_t h[32];
        if (fp32_scale(FMT)) {
            const float s = reinterpret_cast<const float*>(W + scale_off)[pos.scale];
#pragma unroll
            for (int j = 0; j < 32; ++j) h[j] = rn16_code_times_f32(code[j], s);
        } else {
            const _Float16 d = reinterpret_cast<const _Float16*>(W + scale_off)[pos.scale];
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                // exact fp16 code times fp16 scale: one correctly rounded fp16 product
                const _Float16 p = _Float16(float(code[j])) * d;
                h[j] = __builtin_bit_cast(uint16_t, p);
            }
        }
        u32x4* o = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + row * K + int64_t(u) * 32);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            u32x4 t;
            t.x = uint32_t(h[8 * v + 0]) | (uint32_t(h[8 * v + 1]) << 16);
            t.y = uint32_t(h[8 * v + 2]) | (uint32_t(h[8 * v + 3]) << 16);
            t.z = uint32_t(h[8 * v + 4]) | (uint32_t(h[8 * v + 5]) << 16);
            t.w = uint32_t(h[8 * v + 6]) | (uint32_t(h[8 * v + 7]) << 16);
            o[v] = t;
        }
    }
}

// ------------------------------------------------------------ quantize ----
// Load-time block quantization ("oxinfer" page, "How it works": weights are
// block-quantized at load time; "wgpu-llm" page, "INT8 mode": symmetric int8
// with block size 64).  The pages give no rounding rule; the one implemented,
// step by step in IEEE fp32 (correctly rounded divisions, round to nearest
// even):
//   Q8_0:  a = max |w|, d = fp16(a / 127), c = clamp(rint(w / d), -127, 127)
//   Q4_0:  m = first w of largest |w|, d = fp16(m / -8),
//          q = clamp(rint(w / d), -8, 7) + 8
//   int8 block-64: a = max |w|, s = a / 127, c = clamp(rint(w / s), -127, 127)
// A zero scale gives zero weights (code 0, Q4_0 code 8).  One thread per
// block, written straight into the packed tiled layout.
template <int SDT>
__device__ __forceinline__ float source_value(const void* src, int64_t i) {
    if constexpr (SDT == kF32) {
        return static_cast<const float*>(src)[i];
    } else if constexpr (SDT == kF16) {
        return float(static_cast<const _Float16*>(src)[i]);
    } else {
        return __uint_as_float(uint32_t(static_cast<const uint16_t*>(src)[i]) << 16);   // bf16
    }
}

// fp16(v) of an fp32 value that is first materialized as fp32: without the
// empty asm the compiler folds x / -8 and the conversion into one
// v_fma_mixlo_f16(x, -0.125, +0), which turns a -0 quotient into +0.
__device__ __forceinline__ _Float16 to_half(float v) {
    asm volatile("" : "+v"(v));
    return _Float16(v);
}

__device__ __forceinline__ int round_clamp(float v, int lo, int hi) {
    return int(fminf(fmaxf(rintf(v), float(lo)), float(hi)));
}

template <int FMT, int SDT>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const void* __restrict__ src,
                                                            uint8_t* __restrict__ dst, int64_t N,
                                                            int64_t nu, size_t scale_off) {
    constexpr int E = unit_elems(FMT);
    constexpr int P = unit_parts(FMT);
    const int64_t g = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (g >= N * nu) return;
    const int64_t row = g / nu;
    const int64_t u = g - row * nu;
    const int64_t K = nu * E;
    float w[E];
#pragma unroll
    for (int e = 0; e < E; ++e) w[e] = source_value<SDT>(src, row * K + u * E + e);
    const TiledPos pos = tiled_pos(FMT, N, nu, row, u);
    uint8_t q[E];
    if constexpr (fp32_scale(FMT)) {
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) a = fabsf(w[e]) > a ? fabsf(w[e]) : a;
        const float s = a / 127.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) q[e] = uint8_t(int8_t(s == 0.0f ? 0 : round_clamp(w[e] / s, -127, 127)));
        reinterpret_cast<float*>(dst + scale_off)[pos.scale] = s;
    } else {
        _Float16 dh;
        if constexpr (FMT == kQ8_0) {
            float a = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) a = fabsf(w[e]) > a ? fabsf(w[e]) : a;
            dh = to_half(a / 127.0f);
        } else {
            float m = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) m = fabsf(w[e]) > fabsf(m) ? w[e] : m;
            dh = to_half(m / -8.0f);
        }
        const float d = float(dh);
        if constexpr (FMT == kQ8_0) {
#pragma unroll
            for (int e = 0; e < E; ++e) q[e] = uint8_t(int8_t(d == 0.0f ? 0 : round_clamp(w[e] / d, -127, 127)));
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) q[e] = uint8_t(d == 0.0f ? 8 : round_clamp(w[e] / d, -8, 7) + 8);
        }
        reinterpret_cast<_Float16*>(dst + scale_off)[pos.scale] = dh;
    }
    // Codes: Q4_0 byte j = q_j | q_{j+16} << 4 (GGUF order); int8: bytes in order.
    uint32_t b[4 * P];
    if constexpr (FMT == kQ4_0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            b[i] = uint32_t(q[4 * i] | (q[4 * i + 16] << 4)) | (uint32_t(q[4 * i + 1] | (q[4 * i + 17] << 4)) << 8) |
                   (uint32_t(q[4 * i + 2] | (q[4 * i + 18] << 4)) << 16) | (uint32_t(q[4 * i + 3] | (q[4 * i + 19] << 4)) << 24);
    } else {
#pragma unroll
        for (int i = 0; i < 4 * P; ++i)
            b[i] = uint32_t(q[4 * i]) | (uint32_t(q[4 * i + 1]) << 8) | (uint32_t(q[4 * i + 2]) << 16) |
                   (uint32_t(q[4 * i + 3]) << 24);
    }
#pragma unroll
    for (int p = 0; p < P; ++p)
        *reinterpret_cast<u32x4*>(dst + pos.code + size_t(p) * pos.part_stride) =
            u32x4{b[4 * p], b[4 * p + 1], b[4 * p + 2], b[4 * p + 3]};
}

int blocks_for(int64_t n) { return int((n + kThreads - 1) / kThreads); }

}  // namespace

hipError_t launch_repack_gguf(int fmt, const void* src, void* dst, int64_t N, int64_t K,
                              hipStream_t stream) {
    const int64_t nu = K / 32;
    const size_t off = align256(code_plane_bytes(fmt, N, K));
    const uint16_t* s = static_cast<const uint16_t*>(src);
    uint8_t* d = static_cast<uint8_t*>(dst);
    const dim3 grid(blocks_for(N * nu));
    if (fmt == kQ4_0)
        hipLaunchKernelGGL(repack_kernel<kQ4_0>, grid, dim3(kThreads), 0, stream, s, d, N, nu, off);
    else if (fmt == kQ8_0)
        hipLaunchKernelGGL(repack_kernel<kQ8_0>, grid, dim3(kThreads), 0, stream, s, d, N, nu, off);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_pack_planes(int fmt, const void* codes, const void* scales, void* dst, int64_t N,
                              int64_t K, hipStream_t stream) {
    const int64_t nu = K / unit_elems(fmt);
    const size_t off = align256(code_plane_bytes(fmt, N, K));
    const uint8_t* c = static_cast<const uint8_t*>(codes);
    const uint8_t* s = static_cast<const uint8_t*>(scales);
    uint8_t* d = static_cast<uint8_t*>(dst);
    const dim3 grid(blocks_for(N * nu));
    switch (fmt) {
        case kQ4_0: hipLaunchKernelGGL(pack_kernel<kQ4_0>, grid, dim3(kThreads), 0, stream, c, s, d, N, nu, off); break;
        case kQ8_0: hipLaunchKernelGGL(pack_kernel<kQ8_0>, grid, dim3(kThreads), 0, stream, c, s, d, N, nu, off); break;
        case kI8B64: hipLaunchKernelGGL(pack_kernel<kI8B64>, grid, dim3(kThreads), 0, stream, c, s, d, N, nu, off); break;
        case kI8B32: hipLaunchKernelGGL(pack_kernel<kI8B32>, grid, dim3(kThreads), 0, stream, c, s, d, N, nu, off); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_quantize(int fmt, int sdt, const void* src, void* dst, int64_t N, int64_t K,
                           hipStream_t stream) {
    const int64_t nu = K / unit_elems(fmt);
    const size_t off = align256(code_plane_bytes(fmt, N, K));
    uint8_t* d = static_cast<uint8_t*>(dst);
    const dim3 grid(blocks_for(N * nu)), block(kThreads);
#define LQ_QK(F, S) hipLaunchKernelGGL((quantize_kernel<F, S>), grid, block, 0, stream, src, d, N, nu, off)
    switch (fmt * 3 + sdt) {
        case kQ4_0 * 3 + kF32: LQ_QK(kQ4_0, kF32); break;
        case kQ4_0 * 3 + kF16: LQ_QK(kQ4_0, kF16); break;
        case kQ4_0 * 3 + kBF16: LQ_QK(kQ4_0, kBF16); break;
        case kQ8_0 * 3 + kF32: LQ_QK(kQ8_0, kF32); break;
        case kQ8_0 * 3 + kF16: LQ_QK(kQ8_0, kF16); break;
        case kQ8_0 * 3 + kBF16: LQ_QK(kQ8_0, kBF16); break;
        case kI8B64 * 3 + kF32: LQ_QK(kI8B64, kF32); break;
        case kI8B64 * 3 + kF16: LQ_QK(kI8B64, kF16); break;
        case kI8B64 * 3 + kBF16: LQ_QK(kI8B64, kBF16); break;
        case kI8B32 * 3 + kF32: LQ_QK(kI8B32, kF32); break;
        case kI8B32 * 3 + kF16: LQ_QK(kI8B32, kF16); break;
        case kI8B32 * 3 + kBF16: LQ_QK(kI8B32, kBF16); break;
        default: return hipErrorInvalidValue;
    }
#undef LQ_QK
    return hipGetLastError();
}

hipError_t launch_dequant(int fmt, bool to_f16, const void* W, void* out, int64_t N, int64_t K,
                          hipStream_t stream) {
    const int nh = int(K / 32);
    const size_t off = align256(code_plane_bytes(fmt, N, K));
    const uint8_t* w = static_cast<const uint8_t*>(W);
    const dim3 grid(blocks_for(N * nh)), block(kThreads);
#define LQ_DQ(F, H) hipLaunchKernelGGL((dequant_kernel<F, H>), grid, block, 0, stream, w, out, N, nh, off)
    switch (fmt * 2 + (to_f16 ? 1 : 0)) {
        case kQ4_0 * 2 + 0: LQ_DQ(kQ4_0, false); break;
        case kQ4_0 * 2 + 1: LQ_DQ(kQ4_0, true); break;
        case kQ8_0 * 2 + 0: LQ_DQ(kQ8_0, false); break;
        case kQ8_0 * 2 + 1: LQ_DQ(kQ8_0, true); break;
        case kI8B64 * 2 + 0: LQ_DQ(kI8B64, false); break;
        case kI8B64 * 2 + 1: LQ_DQ(kI8B64, true); break;
        case kI8B32 * 2 + 0: LQ_DQ(kI8B32, false); break;
        case kI8B32 * 2 + 1: LQ_DQ(kI8B32, true); break;
        default: return hipErrorInvalidValue;
    }
#undef LQ_DQ
    return hipGetLastError();
}

}  // namespace lq
