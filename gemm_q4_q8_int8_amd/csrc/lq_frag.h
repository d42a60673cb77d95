// Device helpers shared by the matrix-core kernels that take weights straight
// from the packed layout into MFMA operands (multi-token GEMV, prefill GEMM):
// a 4 x 4 dword transpose across the four 16-lane rows of a wave, exact fp16
// fragments of Q4_0 and int8 codes, and activation fragments in the same
// element order.  Not installed.
#pragma once

#include "lq_internal.h"

namespace lq {
namespace frag {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t orv) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(orv));
    return r;
}

// Transpose of the 4 x 4 dwords held by lanes r, r+16, r+32, r+48: on return
// lane (r, j) holds in slot m what lane (r, m) held in slot j.
__device__ __forceinline__ u32x4 xpose(const u32x4 c) {
    const auto a = __builtin_amdgcn_permlane32_swap(c.x, c.z, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(c.y, c.w, false, false);
    const auto lo = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// B fragment of Q4_0 code dword j (bytes 4j..4j+3 of a block) as 8 exact fp16
// values q - 8, elements in the order 4j, 4j+2, 4j+1, 4j+3, 16+4j, 16+4j+2,
// 16+4j+1, 16+4j+3.  A nibble at bits 0-3 of a half under exponent 0x6400 is
// 1024 + q (minus 1032 gives q - 8); at bits 4-7 it is 1024 + 16 q, and
// (1024 + 16 q) / 16 - 72 = q - 8 in one fused multiply-add.  Every step is
// exact.
__device__ __forceinline__ half8_t q4_frag(uint32_t d) {
    const uint32_t kExp = 0x64006400u;
    const half2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
    const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const half2_t off_hi = {(_Float16)-72.0f, (_Float16)-72.0f};
    const uint32_t e = d >> 8;
    const half2_t a = as_h2(and_or(d, 0x000F000Fu, kExp)) - off;
    const half2_t b = as_h2(and_or(e, 0x000F000Fu, kExp)) - off;
    const half2_t c = __builtin_elementwise_fma(as_h2(and_or(d, 0x00F000F0u, kExp)), sixteenth, off_hi);
    const half2_t f = __builtin_elementwise_fma(as_h2(and_or(e, 0x00F000F0u, kExp)), sixteenth, off_hi);
    return __builtin_bit_cast(half8_t, u32x4{as_u32(a), as_u32(b), as_u32(c), as_u32(f)});
}

// B fragment of 8 int8 codes (the 4 bytes of `lo`, then the 4 of `hi`) as
// exact fp16 values in that order.  Flipping each sign bit gives c + 128; a
// byte permute places two of those under 0x64 (fp16 1024 + v) and
// subtracting 1152 leaves the exact codes.
__device__ __forceinline__ half8_t i8_frag(uint32_t lo, uint32_t hi) {
    const half2_t off = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t a = lo ^ 0x80808080u, b = hi ^ 0x80808080u;
    const half2_t p0 = as_h2(__builtin_amdgcn_perm(0x64646464u, a, 0x04010400u)) - off;
    const half2_t p1 = as_h2(__builtin_amdgcn_perm(0x64646464u, a, 0x04030402u)) - off;
    const half2_t p2 = as_h2(__builtin_amdgcn_perm(0x64646464u, b, 0x04010400u)) - off;
    const half2_t p3 = as_h2(__builtin_amdgcn_perm(0x64646464u, b, 0x04030402u)) - off;
    return __builtin_bit_cast(half8_t, u32x4{as_u32(p0), as_u32(p1), as_u32(p2), as_u32(p3)});
}

// A fragment (activations of one token) matching the B fragment's element
// order: lo = x[4j .. 4j+3], hi = x[16+4j .. 16+4j+3] as fp16 pairs.
template <int FMT>
__device__ __forceinline__ half8_t x_frag(const u32x2 lo, const u32x2 hi) {
    if constexpr (FMT == kQ4_0) {
        // (x0, x2), (x1, x3) of each group of four.
        return __builtin_bit_cast(
            half8_t, u32x4{__builtin_amdgcn_perm(lo.y, lo.x, 0x05040100u),
                           __builtin_amdgcn_perm(lo.y, lo.x, 0x07060302u),
                           __builtin_amdgcn_perm(hi.y, hi.x, 0x05040100u),
                           __builtin_amdgcn_perm(hi.y, hi.x, 0x07060302u)});
    } else {
        return __builtin_bit_cast(half8_t, u32x4{lo.x, lo.y, hi.x, hi.y});
    }
}


}  // namespace frag
}  // namespace lq
