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
// One thread handles one block (repack, pack) or 32 weights (dequant).  These kernels run once per weight
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
        if (FMT == kI8B64) s = reinterpret_cast<const float*>(W + scale_off)[pos.scale];
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
        if (FMT == kI8B64) {
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
        default: return hipErrorInvalidValue;
    }
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
        default: return hipErrorInvalidValue;
    }
#undef LQ_DQ
    return hipGetLastError();
}

}  // namespace lq
