// Dequantizing GEMV for decode: y = W x with W in the tiled packed layout
// (Q4_0 / Q8_0 / int8 block-64).
//
// Decode streams every weight once, so the kernel is bound by HBM bandwidth
// ("oxinfer" page, "Performance": decode is memory-bandwidth bound and its
// speed is set by bytes per token).  Design for gfx950:
//   * Lane r of a wave owns row r of a 64-row tile.  The tiled layout stores
//     one 16-byte part of one unit (scale block) for all 64 rows of a tile as
//     one contiguous 1 KB run, so every code load of a wave is one coalesced
//     16-byte-per-lane non-temporal load, and each lane accumulates its own
//     row: no cross-lane reduction at all.
//   * The activations are the same for every lane, so they are read with
//     scalar loads (s_load into SGPRs, served by the scalar cache) and feed
//     the vector FMAs as scalar operands: no LDS staging, no barrier, no VGPRs.
//   * A workgroup of 4 waves (16 for launches of small matrices) takes one
//     tile and splits its units among its waves; the partial sums meet in
//     LDS in a fixed order.  When the matrices
//     of a launch have too few tiles to fill the chip (one 2048-row matrix is
//     32 tiles), K is also split across S workgroups per tile: each writes
//     its slice's sums to the caller's workspace and bumps the tile's
//     arrival counter; the last one to arrive adds the S slices in slice
//     order (deterministic) and writes y.
//   * Each wave issues the loads of a batch of UNR units before it computes
//     any of them (all in flight at once, consumed in load order).  UNR is
//     chosen per launch so that the batches split a wave's units evenly: a
//     slot past the wave's last unit still loads and computes (a select then
//     leaves the sums unchanged), since per-slot branches let the compiler sink loads below
//     the first slot's arithmetic.  Q4_0 (most arithmetic per byte) takes
//     up to 8 units per batch, Q8_0 2 and int8 block-64 1 (2 in launches with
//     few waves): with the waves resident per SIMD, larger batches were
//     measured slower.
//   * Q4_0 nibbles become exact fp16 values (q - 8) with one v_and_or_b32
//     (nibble into an fp16 mantissa under exponent 2^10) and one v_pk_add_f16
//     per two weights.  fp32 activations: v_fma_mix_f32 multiplies that fp16
//     by the fp32 activation into an fp32 sum.  fp16 activations: v_dot2 of
//     two fp16 weights with two fp16 activations into an fp32 sum.
//   * int8 codes: sign-extending SDWA byte selects into v_cvt_f32_i32 and an
//     fp32 FMA (fp32 activations), or a byte permute into fp16 pairs and
//     v_dot2 (fp16 activations).
//   * The block scale multiplies the unit's partial sum once per block.
#include "lq_splitk.h"

#include <type_traits>

namespace lq {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Activations are read through the constant address space so that uniform
// indices turn into scalar loads.
typedef const __attribute__((address_space(4))) float* cf32_p;
typedef const __attribute__((address_space(4))) uint32_t* cu32_p;

__device__ __forceinline__ half2_t as_half2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// (a & mask) | orv in one VALU op.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t orv) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(orv));
    return r;
}

// Q4_0 code dword d (bytes 4i..4i+3 of a block) as four exact fp16 pairs.
// Byte j holds element j (low nibble) and element j + 16 (high nibble).  A
// nibble at bits 0-3 of a half, ORed under 0x6400, is the fp16 value 1024 + q;
// at bits 4-7 it is 1024 + 16q.  Subtracting 1032 (or 1152) gives q - 8 (or
// 16 (q - 8)) exactly:
//   t0 = elements (4i, 4i+2), t2 = (4i+1, 4i+3),
//   t1 = 16 x elements (16+4i, 16+4i+2), t3 = 16 x (16+4i+1, 16+4i+3).
struct Q4Pairs {
    half2_t t0, t1, t2, t3;
};
__device__ __forceinline__ Q4Pairs q4_pairs(uint32_t d) {
    const uint32_t kExp = 0x64006400u;
    const half2_t lo_off = {(_Float16)1032.0f, (_Float16)1032.0f};
    const half2_t hi_off = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t e = d >> 8;
    Q4Pairs p;
    p.t0 = as_half2(and_or(d, 0x000F000Fu, kExp)) - lo_off;
    p.t1 = as_half2(and_or(d, 0x00F000F0u, kExp)) - hi_off;
    p.t2 = as_half2(and_or(e, 0x000F000Fu, kExp)) - lo_off;
    p.t3 = as_half2(and_or(e, 0x00F000F0u, kExp)) - hi_off;
    return p;
}

// The same four pairs in element order, for fp16 activations: a byte permute
// puts bytes (4i, 4i+1) and (4i+2, 4i+3) of the dword under 0x64, and one
// mask per pair keeps the low or the high nibble:
//   t0 = elements (4i, 4i+1), t2 = (4i+2, 4i+3),
//   t1 = 16 x elements (16+4i, 16+4i+1), t3 = 16 x (16+4i+2, 16+4i+3).
// One more vector instruction per dword than q4_pairs, but each pair then
// meets an activation dword as loaded: the pairs q4_pairs gives needed four
// scalar packs per dword and token, and the scalar unit (one per CU) was the
// limit of the fp16 launches (two-token LM head: 371 scalar instructions
// per wave).
__device__ __forceinline__ Q4Pairs q4_pairs_seq(uint32_t d) {
    const half2_t lo_off = {(_Float16)1032.0f, (_Float16)1032.0f};
    const half2_t hi_off = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t a = __builtin_amdgcn_perm(0x64646464u, d, 0x04010400u);   // [b0, 64, b1, 64]
    const uint32_t b = __builtin_amdgcn_perm(0x64646464u, d, 0x04030402u);   // [b2, 64, b3, 64]
    Q4Pairs p;
    p.t0 = as_half2(a & 0x640F640Fu) - lo_off;
    p.t1 = as_half2(a & 0x64F064F0u) - hi_off;
    p.t2 = as_half2(b & 0x640F640Fu) - lo_off;
    p.t3 = as_half2(b & 0x64F064F0u) - hi_off;
    return p;
}

// The 32 fp32 activations of one unit, wave-uniform, as two 64-byte scalar
// loads (x is 16-byte aligned; a scalar load needs only dword alignment, and
// the type says no more).  Eight-dword loads with a wait per pair cost the
// Q8_0 decoder layer 0.26 us (12.89 -> 12.63 us with these).
typedef float f32x16v __attribute__((ext_vector_type(16), aligned(4)));
typedef const __attribute__((address_space(4))) f32x16v* cf32x16_p;
__device__ __forceinline__ void load_x32(cf32_p x, float (&o)[32]) {
    const f32x16v a = *reinterpret_cast<cf32x16_p>(x), b = *reinterpret_cast<cf32x16_p>(x + 16);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        o[k] = a[k];
        o[16 + k] = b[k];
    }
}
// The same for 32 fp16 activations (16 dwords, one 64-byte load).
typedef uint32_t u32x16v __attribute__((ext_vector_type(16), aligned(4)));
typedef const __attribute__((address_space(4))) u32x16v* cu32x16_p;
__device__ __forceinline__ void load_x16(cu32_p x, uint32_t (&o)[16]) {
    const u32x16v a = *reinterpret_cast<cu32x16_p>(x);
#pragma unroll
    for (int k = 0; k < 16; ++k) o[k] = a[k];
}

// sum_e (q_e - 8) x_e over one Q4_0 block, fp32 activations in SGPRs.  The
// high-nibble sum is 16x too large and is scaled by 1/16 (exact) at the end.
__device__ __forceinline__ float dot_q4_0_f32(const u32x4 c, cf32_p x0) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    float x[32];
    load_x32(x0, x);
    float s_lo = 0.0f, s_hi = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const Q4Pairs p = q4_pairs(w[i]);
        s_lo = __builtin_fmaf((float)p.t0.x, x[4 * i + 0], s_lo);
        s_lo = __builtin_fmaf((float)p.t2.x, x[4 * i + 1], s_lo);
        s_lo = __builtin_fmaf((float)p.t0.y, x[4 * i + 2], s_lo);
        s_lo = __builtin_fmaf((float)p.t2.y, x[4 * i + 3], s_lo);
        s_hi = __builtin_fmaf((float)p.t1.x, x[16 + 4 * i + 0], s_hi);
        s_hi = __builtin_fmaf((float)p.t3.x, x[16 + 4 * i + 1], s_hi);
        s_hi = __builtin_fmaf((float)p.t1.y, x[16 + 4 * i + 2], s_hi);
        s_hi = __builtin_fmaf((float)p.t3.y, x[16 + 4 * i + 3], s_hi);
    }
    return __builtin_fmaf(s_hi, 0.0625f, s_lo);
}

// Same sum with fp16 activations for MT tokens: x[t] holds token t's pairs
// (x_2i, x_2i+1).  The nibbles are unpacked once for all tokens.
template <int MT>
__device__ __forceinline__ void dot_q4_0_f16(const u32x4 c, const cu32_p (&x)[MT], float (&out)[MT]) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    float s_lo[MT], s_hi[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) s_lo[t] = s_hi[t] = 0.0f;
    uint32_t xv[MT][16];
#pragma unroll
    for (int t = 0; t < MT; ++t) load_x16(x[t], xv[t]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const Q4Pairs p = q4_pairs_seq(w[i]);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            s_lo[t] = __builtin_amdgcn_fdot2(p.t0, as_half2(xv[t][2 * i]), s_lo[t], false);          // x 4i, 4i+1
            s_lo[t] = __builtin_amdgcn_fdot2(p.t2, as_half2(xv[t][2 * i + 1]), s_lo[t], false);      // x 4i+2, 4i+3
            s_hi[t] = __builtin_amdgcn_fdot2(p.t1, as_half2(xv[t][8 + 2 * i]), s_hi[t], false);      // x 16+4i ..
            s_hi[t] = __builtin_amdgcn_fdot2(p.t3, as_half2(xv[t][8 + 2 * i + 1]), s_hi[t], false);
        }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) out[t] = __builtin_fmaf(s_hi[t], 0.0625f, s_lo[t]);
}

// Signed byte n of a dword to fp32 in one VALU op (SDWA byte select with
// sign extension).  Written out so the compiler cannot split each loaded
// dword into four shifted copies ahead of use.
#define LQ_SBYTE_TO_F32(NAME, SEL)                                                       \
    __device__ __forceinline__ float NAME(uint32_t d) {                                  \
        float r;                                                                         \
        asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:" SEL \
            : "=v"(r)                                                                    \
            : "v"(d));                                                                   \
        return r;                                                                        \
    }
LQ_SBYTE_TO_F32(sbyte0, "BYTE_0")
LQ_SBYTE_TO_F32(sbyte1, "BYTE_1")
LQ_SBYTE_TO_F32(sbyte2, "BYTE_2")
LQ_SBYTE_TO_F32(sbyte3, "BYTE_3")
#undef LQ_SBYTE_TO_F32

// sum_e c_e x_e over 32 int8 codes (two 16-byte parts, element order), fp32
// activations in SGPRs.
__device__ __forceinline__ float dot_i8_f32(const u32x4 c0, const u32x4 c1, cf32_p x0) {
    const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    float x[32];
    load_x32(x0, x);
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t d = w[i];
        s0 = __builtin_fmaf(sbyte0(d), x[4 * i + 0], s0);
        s1 = __builtin_fmaf(sbyte1(d), x[4 * i + 1], s1);
        s0 = __builtin_fmaf(sbyte2(d), x[4 * i + 2], s0);
        s1 = __builtin_fmaf(sbyte3(d), x[4 * i + 3], s1);
    }
    return s0 + s1;
}

// Same with fp16 activations, MT tokens.  Flipping the sign bit of each
// byte gives c + 128 in 0..255; a byte permute puts two of those under 0x64
// (fp16 1024 + v) and subtracting 1152 leaves the exact codes as an fp16
// pair, shared by all tokens.
template <int MT>
__device__ __forceinline__ void dot_i8_f16(const u32x4 c0, const u32x4 c1, const cu32_p (&x)[MT], int xoff,
                                           float (&out)[MT]) {
    const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const half2_t off = {(_Float16)1152.0f, (_Float16)1152.0f};
    float s0[MT], s1[MT];
    uint32_t xv[MT][16];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        s0[t] = s1[t] = 0.0f;
        load_x16(x[t] + xoff, xv[t]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t u = w[i] ^ 0x80808080u;
        const half2_t p01 = as_half2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - off;
        const half2_t p23 = as_half2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - off;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            s0[t] = __builtin_amdgcn_fdot2(p01, as_half2(xv[t][2 * i]), s0[t], false);
            s1[t] = __builtin_amdgcn_fdot2(p23, as_half2(xv[t][2 * i + 1]), s1[t], false);
        }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) out[t] = s0[t] + s1[t];
}

template <int FMT>
struct Unit {
    static constexpr int P = unit_parts(FMT);
    u32x4 c[P];
    uint32_t s;   // raw scale bits (fp16 in the low half, or fp32)
};

// scale * sum over unit u of code * x, added to acc[t] for each of the MT
// tokens (token t's activations start xs 32-bit words after token 0's; MT > 1
// only with fp16 activations).  keep is false for a slot past the wave's last
// unit: the sums are then left as they were (a select, so a re-read unit
// with an infinite or NaN scale changes nothing).
template <int FMT, int XDT, int MT>
__device__ __forceinline__ void unit_fma(const Unit<FMT>& b, const void* xv, size_t xs, int u, bool keep,
                                         float (&acc)[MT]) {
    constexpr int E = unit_elems(FMT);
    float dot[MT];
    if constexpr (XDT == kF32) {
        static_assert(MT == 1, "several tokens take fp16 activations");
        const cf32_p x = (cf32_p)(xv) + size_t(u) * E;
        if constexpr (FMT == kQ4_0) dot[0] = dot_q4_0_f32(b.c[0], x);
        else if constexpr (unit_parts(FMT) == 2) dot[0] = dot_i8_f32(b.c[0], b.c[1], x);
        else dot[0] = dot_i8_f32(b.c[0], b.c[1], x) + dot_i8_f32(b.c[2], b.c[3], x + 32);
    } else {
        cu32_p x[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) x[t] = (cu32_p)(xv) + size_t(t) * xs + size_t(u) * (E / 2);
        if constexpr (FMT == kQ4_0) {
            dot_q4_0_f16<MT>(b.c[0], x, dot);
        } else if constexpr (unit_parts(FMT) == 2) {
            dot_i8_f16<MT>(b.c[0], b.c[1], x, 0, dot);
        } else {
            float d2[MT];
            dot_i8_f16<MT>(b.c[0], b.c[1], x, 0, dot);
            dot_i8_f16<MT>(b.c[2], b.c[3], x, 16, d2);
#pragma unroll
            for (int t = 0; t < MT; ++t) dot[t] += d2[t];
        }
    }
    float d;
    if constexpr (fp32_scale(FMT)) d = __uint_as_float(b.s);
    else d = (float)__builtin_bit_cast(_Float16, uint16_t(b.s));
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const float f = __builtin_fmaf(d, dot[t], acc[t]);
        acc[t] = keep ? f : acc[t];
    }
}

// Largest batch of units one wave loads before computing them (register
// budget: the codes of a batch stay live).  Q8_0 / int8 block-32: one-unit
// loads of 2 KB per wave, 4 per batch for one or two tokens (the Q8_0 layer
// launch: 13.92 -> 13.73-13.84 us against batches of 2; the layer at two
// tokens 15.04 -> 14.49 us), 2 for more tokens (four tokens with batches of
// 4: 16.95 -> 18.11 us).
constexpr int unroll_cap(int fmt) { return fmt == kQ4_0 ? LQ_GEMV_UNR_Q4 : (fmt == kI8B64 ? LQ_GEMV_UNR_I8 : LQ_GEMV_UNR_Q8); }
inline int unroll_cap(int fmt, int mt) {
    return (fmt == kQ8_0 || fmt == kI8B32) && mt > 2 ? LQ_GEMV_UNR_Q8_TOKENS : unroll_cap(fmt);
}

// W waves per workgroup split a tile's K slice W ways (4, or 16 for
// launches whose matrices would otherwise split K across 4+ workgroups: the
// split then stays inside the workgroup and needs no split-K round trips).
// Each wave loads UNR units, then computes them, until its units are done.
// MT tokens (1, or 2 with fp16 activations) share every weight load: x holds
// MT rows of K values, y MT rows of N outputs.
template <int FMT, int XDT, int W, int UNR, int MT>
__global__ __launch_bounds__(64 * W) void gemv_kernel(const GemvArgs a) {
    constexpr int P = unit_parts(FMT);
    constexpr int UB = unit_bytes(FMT);
    constexpr int SB = scale_bytes(FMT);
    __shared__ float red[MT][W][kTileRows];

    const int bid = blockIdx.x;
    const GemvDesc& D = a.d[find_matrix(a.wg0, bid)];
    const int N = D.N, nu = D.nu, S = D.S;
    const int local = bid - D.wg0;
    // The fields the first loads need, all in one scalar round trip (the
    // empty asm keeps the compiler from issuing the pointers' loads after
    // the others have returned).
    const uint8_t* const dcodes = D.codes;
    const uint8_t* const dscales = D.scales;
    const uint32_t dtb = D.tile_bytes;
    asm volatile("" : : "s"(dcodes), "s"(dscales), "s"(dtb), "s"(N), "s"(nu), "s"(S), "s"(local));
    // Units [sa, sb) of this workgroup: slice `slice` of S.  (Unsplit
    // matrices skip the divisions: with a few units per wave they are a
    // noticeable share of the wave's scalar work.)
    int tile = local, slice = 0, sa = 0, sb = nu;
    if (S > 1) {
        tile = int(uint32_t(local) / uint32_t(S));
        slice = local - tile * S;
        slice_units(nu, S, slice, sa, sb);
    }
    const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    const int r = int(threadIdx.x) & 63;
    const int nr = min(kTileRows, N - tile * kTileRows);
    const int rc = min(r, nr - 1);   // lanes past the last row re-read it and store nothing

    // Units [ua, ub) of this wave: part w of W of the slice (unsigned
    // arithmetic: W is a power of two, so these are shifts).
    const int ua = __builtin_amdgcn_readfirstlane(sa + int(uint32_t(sb - sa) * uint32_t(w) / W));
    const int ub = __builtin_amdgcn_readfirstlane(sa + int(uint32_t(sb - sa) * uint32_t(w + 1) / W));

    // Uniform tile bases plus 32-bit per-lane offsets (scalar base + vector
    // offset addressing).  A tile's scale bytes are its code bytes times
    // SB / UB (1/8 or 1/16).
    static_assert(UB % SB == 0 && ((UB / SB) & (UB / SB - 1)) == 0, "scale / code ratio");
    const uint64_t tcode = uint64_t(uint32_t(tile)) * dtb;
    const uint8_t* cbase = dcodes + tcode;
    const uint8_t* sbase = dscales + tcode / (UB / SB);
    const uint32_t c_lane = uint32_t(rc) * 16u;
    const uint32_t c_unit = uint32_t(nr) * UB;
    const uint32_t c_part = uint32_t(nr) * 16u;
    const uint32_t s_lane = uint32_t(rc) * SB;
    const uint32_t s_unit = uint32_t(nr) * SB;
    const void* x = D.x;
    const size_t xs = size_t(nu) * (unit_elems(FMT) / 2);   // 32-bit words per fp16 token row

    float acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = 0.0f;
    for (int u = ua; u < ub; u += UNR) {
        // fp16 scales stream past the caches like the codes: as cached
        // 2-byte loads they cost the Q8_0 decoder layer 7 % of its time.
        // (The fp32 scales of int8 block-64 measured 1 % faster cached.)
        Unit<FMT> b[UNR];
        auto load_scale = [&](int k) {
            const uint32_t so = uint32_t(min(u + k, ub - 1)) * s_unit + s_lane;
            if constexpr (SB == 2)
                b[k].s = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(sbase + so));
            else
                b[k].s = *reinterpret_cast<const uint32_t*>(sbase + so);
        };
        auto load_codes = [&](int k) {
            const uint32_t co = uint32_t(min(u + k, ub - 1)) * c_unit + c_lane;
#pragma unroll
            for (int p = 0; p < P; ++p)
                b[k].c[p] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4*>(cbase + co + uint32_t(p) * c_part));
        };
        if constexpr (scales_first(FMT)) {
#pragma unroll
            for (int k = 0; k < UNR; ++k) load_scale(k);
#pragma unroll
            for (int k = 0; k < UNR; ++k) load_codes(k);
        } else {
#pragma unroll
            for (int k = 0; k < UNR; ++k) {
                load_codes(k);
                load_scale(k);
            }
        }
        // Every load of the batch is issued before any of its data is used,
        // and every slot is computed: a branch per slot let the compiler sink
        // loads below the first slot's arithmetic.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < UNR; ++k)
            unit_fma<FMT, XDT, MT>(b[k], x, xs, min(u + k, ub - 1), u + k < ub, acc);
    }

#pragma unroll
    for (int t = 0; t < MT; ++t) red[t][w][r] = acc[t];
    __syncthreads();
    if (w != 0) return;
    float v[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        v[t] = 0.0f;
#pragma unroll
        for (int i = 0; i < W; i += 4)
            v[t] += (red[t][i][r] + red[t][i + 1][r]) + (red[t][i + 2][r] + red[t][i + 3][r]);
    }
    const size_t row = size_t(tile) * kTileRows + size_t(r);
    if (S == 1) {
        if (r < nr) {
#pragma unroll
            for (int t = 0; t < MT; ++t) D.y[size_t(t) * N + row] = v[t];
        }
        return;
    }
    // Split K: publish this slice, then the last arrival sums all slices in
    // slice order (lq_splitk.h).  Slice j of token t sits at rows
    // (j * MT + t) * pitch.
    const size_t pitch = size_t(D.tiles) * kTileRows;
#pragma unroll
    for (int t = 0; t < MT; ++t) splitk_put(&D.part[(size_t(slice) * MT + t) * pitch + row], v[t]);
    splitk_publish();
    uint32_t last = 0;
    if (r == 0) last = splitk_arrive(&D.cnt[tile], a.tag, S) ? 1u : 0u;
    last = __builtin_amdgcn_readfirstlane(last);
    if (!last) return;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const float y = sum_slices(D.part + size_t(t) * pitch + row, MT * pitch, S);
        if (r < nr) D.y[size_t(t) * N + row] = y;
    }
}

// 16 weights (one code part) times 16 activations held in VGPRs: the sub-tile
// kernel's lanes each take one part of a unit, so their activations differ
// between lane groups and cannot sit in SGPRs.
__device__ __forceinline__ float dot16_i8(const u32x4 c, const u32x4 (&x)[2]) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    const uint32_t xx[8] = {x[0].x, x[0].y, x[0].z, x[0].w, x[1].x, x[1].y, x[1].z, x[1].w};
    const half2_t off = {(_Float16)1152.0f, (_Float16)1152.0f};
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t u = w[i] ^ 0x80808080u;
        const half2_t p01 = as_half2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - off;
        const half2_t p23 = as_half2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - off;
        s0 = __builtin_amdgcn_fdot2(p01, as_half2(xx[2 * i]), s0, false);
        s1 = __builtin_amdgcn_fdot2(p23, as_half2(xx[2 * i + 1]), s1, false);
    }
    return s0 + s1;
}
__device__ __forceinline__ float dot16_i8(const u32x4 c, const f32x4 (&x)[4]) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t d = w[i];
        s0 = __builtin_fmaf(sbyte0(d), x[i].x, s0);
        s1 = __builtin_fmaf(sbyte1(d), x[i].y, s1);
        s0 = __builtin_fmaf(sbyte2(d), x[i].z, s0);
        s1 = __builtin_fmaf(sbyte3(d), x[i].w, s1);
    }
    return s0 + s1;
}

// Sub-tile GEMV (Q8_0 and int8 block-64) for launches of few 64-row tiles
// (at most one workgroup per CU after the split below), e.g. one decoder
// layer's q/k/v or o projection alone: each tile is split across P workgroups by rows instead of across
// workgroups by K, so P times as many CUs stream it and no partial sum
// leaves its workgroup.  Workgroup (tile, sub) owns rows sub * RPW .. + RPW
// of the tile (RPW = 64 / P, P = 2 or 4 code parts per unit); lane l takes
// row l % RPW and part l / RPW (16 weights) of each unit, so a wave's load is
// still P whole pieces of the unit's contiguous runs.  The 16 waves split
// the units; the part and wave sums of a row are added in LDS in a fixed
// order.  MT tokens (fp16 activations when MT > 1) share the weight loads;
// each token's arithmetic is the same as with MT = 1, and a slot past a
// wave's last unit leaves the sums untouched, so the batch size never
// changes a result.
template <int FMT, int XDT, int UNR, int MT>
__global__ __launch_bounds__(1024) void gemv_sub_kernel(const GemvArgs a) {
    constexpr int W = 16;
    constexpr int P = unit_parts(FMT);
    static_assert(P > 1, "rows are split by code part");
    static_assert(MT == 1 || XDT == kF16, "several tokens take fp16 activations");
    constexpr int RPW = kTileRows / P;
    constexpr int E = unit_elems(FMT);
    constexpr int UB = unit_bytes(FMT);
    constexpr int SB = scale_bytes(FMT);
    __shared__ float red[MT][W][kTileRows];

    const int bid = blockIdx.x;
    const GemvDesc& D = a.d[find_matrix(a.wg0, bid)];
    const int N = D.N, nu = D.nu;
    const int local = bid - D.wg0;
    // Every descriptor field the first loads need, in one scalar round trip
    // (as in gemv_kernel: these launches are small, so the prologue's
    // latency is a large part of them).
    const uint8_t* const dcodes = D.codes;
    const uint8_t* const dscales = D.scales;
    const void* const dx = D.x;
    const uint32_t dtb = D.tile_bytes;
    asm volatile("" : : "s"(dcodes), "s"(dscales), "s"(dx), "s"(dtb), "s"(N), "s"(nu), "s"(local));
    const int tile = int(uint32_t(local) / P);
    const int sub = local - tile * P;
    const int nr = min(kTileRows, N - tile * kTileRows);
    if (sub * RPW >= nr) return;   // whole workgroup: past the last row of a ragged tile
    const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    const int l = int(threadIdx.x) & 63;
    const int p = l / RPW;
    const int rr = sub * RPW + (l - p * RPW);   // row within the tile
    const int rc = min(rr, nr - 1);              // rows past the last re-read it and store nothing
    const int ua = __builtin_amdgcn_readfirstlane(int(uint32_t(nu) * uint32_t(w) / W));
    const int ub = __builtin_amdgcn_readfirstlane(int(uint32_t(nu) * uint32_t(w + 1) / W));

    const uint64_t tcode = uint64_t(uint32_t(tile)) * dtb;   // tile base; scales: SB / UB of it
    const uint8_t* cbase = dcodes + tcode;
    const uint8_t* sbase = dscales + tcode / (UB / SB);
    const uint32_t c_lane = uint32_t(p) * uint32_t(nr) * 16u + uint32_t(rc) * 16u;
    const uint32_t c_unit = uint32_t(nr) * UB;
    const uint32_t s_lane = uint32_t(rc) * SB;
    const uint32_t s_unit = uint32_t(nr) * SB;
    constexpr int XB = XDT == kF32 ? 4 : 2;    // bytes per activation
    constexpr int XV = XB;                     // 16-byte loads per 16 activations
    using XT = typename std::conditional<XDT == kF32, f32x4, u32x4>::type;
    const size_t xrow = size_t(nu) * E * XB / 16;   // one token's activations, in 16-byte units
    const XT* xb = reinterpret_cast<const XT*>(static_cast<const uint8_t*>(dx) + size_t(p) * 16 * XB);

    float acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = 0.0f;
    for (int u = ua; u < ub; u += UNR) {
        u32x4 c[UNR];
        uint32_t sc[UNR];
        XT x[UNR][MT][XV];
#pragma unroll
        for (int k = 0; k < UNR; ++k) {   // scales first (scales_first: P > 1 here)
            const uint32_t so = uint32_t(min(u + k, ub - 1)) * s_unit + s_lane;
            if constexpr (SB == 2)
                sc[k] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(sbase + so));
            else
                sc[k] = *reinterpret_cast<const uint32_t*>(sbase + so);
        }
#pragma unroll
        for (int k = 0; k < UNR; ++k) {
            const uint32_t uu = uint32_t(min(u + k, ub - 1));
            c[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(cbase + uu * c_unit + c_lane));
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int v = 0; v < XV; ++v) x[k][t][v] = xb[size_t(t) * xrow + size_t(uu) * (E / 16) * XV + v];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < UNR; ++k) {
            float d;
            if constexpr (SB == 4) d = __uint_as_float(sc[k]);
            else d = (float)__builtin_bit_cast(_Float16, uint16_t(sc[k]));
            const bool keep = u + k < ub;
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const float f = __builtin_fmaf(d, dot16_i8(c[k], x[k][t]), acc[t]);
                acc[t] = keep ? f : acc[t];
            }
        }
    }

#pragma unroll
    for (int t = 0; t < MT; ++t) red[t][w][l] = acc[t];
    __syncthreads();
    if (w != 0 || l >= RPW) return;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        float v = 0.0f;
#pragma unroll
        for (int q = 0; q < P; ++q)
#pragma unroll
            for (int i = 0; i < W; i += 4)
                v += (red[t][i][q * RPW + l] + red[t][i + 1][q * RPW + l]) +
                     (red[t][i + 2][q * RPW + l] + red[t][i + 3][q * RPW + l]);
        if (rr < nr) D.y[size_t(t) * N + size_t(tile) * kTileRows + size_t(rr)] = v;
    }
}

template <int FMT, int XDT, int UNR, int MT>
hipError_t launch_sub_unr(int unr, const GemvArgs& a, hipStream_t stream) {
    if constexpr (UNR > 1) {
        if (unr < UNR) return launch_sub_unr<FMT, XDT, UNR - 1, MT>(unr, a, stream);
    }
    hipLaunchKernelGGL((gemv_sub_kernel<FMT, XDT, UNR, MT>), dim3(unsigned(a.total_wgs)), dim3(1024u), 0, stream, a);
    return hipGetLastError();
}

template <int FMT, int XDT, int W, int UNR, int MT>
hipError_t launch_unr(int unr, const GemvArgs& a, hipStream_t stream) {
    if constexpr (UNR > 1) {
        if (unr < UNR) return launch_unr<FMT, XDT, W, UNR - 1, MT>(unr, a, stream);
    }
    hipLaunchKernelGGL((gemv_kernel<FMT, XDT, W, UNR, MT>), dim3(unsigned(a.total_wgs)), dim3(64u * W), 0,
                       stream, a);
    return hipGetLastError();
}

// Batch size of a launch: its waves have at most u units (ceil(ceil(nu / S)
// / W)); they run in ceil(u / cap) batches of ceil(u / batches) units, so
// that no batch loads and computes many slots past a wave's last unit.  A
// launch of fewer than kFewWaves waves (under about four per SIMD: a small
// matrix on its own, e.g. one decoder layer's q/k/v or o) has too few loads
// in flight with one-unit batches; it takes batches of at least two units.
constexpr int64_t kFewWaves = 4096;
int launch_unroll(int fmt, int mt, int waves, const GemvArgs& a) {
    int u = 1;
    for (int i = 0; i < a.count; ++i) {
        const int slice = (a.d[i].nu + a.d[i].S - 1) / a.d[i].S;
        u = max(u, (slice + waves - 1) / waves);
    }
    int cap = unroll_cap(fmt, mt);
    if (int64_t(a.total_wgs) * waves < kFewWaves) cap = max(cap, 2);
    const int batches = (u + cap - 1) / cap;
    return (u + batches - 1) / batches;
}

template <int FMT, int MT>
hipError_t launch_tokens(int waves, int mt, int unr, const GemvArgs& a, hipStream_t stream) {
    if constexpr (MT > 2) {
        if (mt < MT) return launch_tokens<FMT, MT - 1>(waves, mt, unr, a, stream);
    }
    constexpr int CAP = unroll_cap(FMT) > 2 ? unroll_cap(FMT) : 2;
    if (waves == 16) return launch_unr<FMT, kF16, 16, CAP, MT>(unr, a, stream);
    return launch_unr<FMT, kF16, 4, CAP, MT>(unr, a, stream);
}

template <int FMT>
hipError_t launch_fmt(int xdt, int waves, int mt, const GemvArgs& a, hipStream_t stream) {
    constexpr int CAP = unroll_cap(FMT) > 2 ? unroll_cap(FMT) : 2;
    const int unr = launch_unroll(FMT, mt, waves, a);
    if (mt > 1) {
        if (xdt != kF16 || mt > gemv_max_tokens(FMT)) return hipErrorInvalidValue;
        return launch_tokens<FMT, gemv_max_tokens(FMT)>(waves, mt, unr, a, stream);
    }
    if (mt != 1) return hipErrorInvalidValue;
    if (waves == 16) {
        if (xdt == kF32) return launch_unr<FMT, kF32, 16, CAP, 1>(unr, a, stream);
        return launch_unr<FMT, kF16, 16, CAP, 1>(unr, a, stream);
    }
    if (xdt == kF32) return launch_unr<FMT, kF32, 4, CAP, 1>(unr, a, stream);
    return launch_unr<FMT, kF16, 4, CAP, 1>(unr, a, stream);
}

// Units a sub-tile wave loads before computing them: a launch's waves have
// at most u = ceil(nu / 16) units, run in equal batches of at most 4 (one
// token) or 2 (several: their activations take the registers).
template <int FMT, int MT>
hipError_t launch_sub_tokens(int xdt, int mt, const GemvArgs& a, hipStream_t stream) {
    if constexpr (MT > 1) {
        if (mt < MT) return launch_sub_tokens<FMT, MT - 1>(xdt, mt, a, stream);
    }
    constexpr int CAP = MT == 1 ? LQ_GEMV_SUB_UNR : 2;
    int u = 1;
    for (int i = 0; i < a.count; ++i) u = max(u, (a.d[i].nu + 15) / 16);
    const int batches = (u + CAP - 1) / CAP;
    const int unr = (u + batches - 1) / batches;
    if constexpr (MT == 1) {
        if (xdt == kF32) return launch_sub_unr<FMT, kF32, CAP, 1>(unr, a, stream);
    }
    return launch_sub_unr<FMT, kF16, CAP, MT>(unr, a, stream);
}

}  // namespace

hipError_t launch_gemv_sub(int fmt, int xdt, int mt, const GemvArgs& a, hipStream_t stream) {
    if (mt < 1 || mt > gemv_max_tokens(fmt) || (mt > 1 && xdt != kF16)) return hipErrorInvalidValue;
    switch (fmt) {
        case kQ8_0: return launch_sub_tokens<kQ8_0, gemv_max_tokens(kQ8_0)>(xdt, mt, a, stream);
        case kI8B64: return launch_sub_tokens<kI8B64, gemv_max_tokens(kI8B64)>(xdt, mt, a, stream);
        case kI8B32: return launch_sub_tokens<kI8B32, gemv_max_tokens(kI8B32)>(xdt, mt, a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv(int fmt, int xdt, int waves, int mt, const GemvArgs& a, hipStream_t stream) {
    if (waves != 4 && waves != 16) return hipErrorInvalidValue;
    switch (fmt) {
        case kQ4_0: return launch_fmt<kQ4_0>(xdt, waves, mt, a, stream);
        case kQ8_0: return launch_fmt<kQ8_0>(xdt, waves, mt, a, stream);
        case kI8B64: return launch_fmt<kI8B64>(xdt, waves, mt, a, stream);
        case kI8B32: return launch_fmt<kI8B32>(xdt, waves, mt, a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lq
