// Dequantizing GEMV for decode: y = W x with W in the packed Q4_0 / Q8_0 /
// int8-block-64 layout.
//
// Decode streams every weight once, so the kernel is bound by HBM bandwidth
// ("oxinfer" page, "Performance": decode is memory-bandwidth bound and its
// speed is set by bytes per token).  Design for gfx950:
//   * A team of TP lanes (16..256) works on one row at a time.  Lane t of a
//     team owns the 32-weight units t, t + TP, ... of every row it touches and
//     keeps those activations in VGPRs for the whole kernel, so x is read from
//     L2 once per workgroup and never re-read per row.
//   * Each lane issues one 128-bit load per unit and row (two for int8
//     codes); consecutive lanes read consecutive 16-byte blocks, so a wave's
//     load covers one contiguous span of the code plane.  All loads of an
//     iteration (RPI rows x UPL units) are issued before any arithmetic.
//   * Q4_0 nibbles become exact fp16 values (q - 8) with one v_and_or_b32
//     (nibble into an fp16 mantissa under exponent 2^10) and one v_pk_add_f16
//     per two weights; v_fma_mix_f32 then multiplies that fp16 by the fp32
//     activation into an fp32 accumulator.  About 2.1 VALU ops per weight.
//   * int8 codes use sign-extending SDWA byte selects into v_cvt_f32_i32 and an
//     fp32 FMA: 2 VALU ops per weight.
//   * The block scale multiplies the unit's partial sum once (per block, not
//     per weight).  Partial sums of a row are combined across the team with
//     a transposed butterfly: each halving step exchanges half of the rows'
//     partials, so RPI rows cost about RPI + log2(TP) shuffles instead of
//     RPI * log2(TP).  Teams wider than a wave finish through LDS.
#include "lq_internal.h"

namespace lq {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half2_t as_half2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// (a & mask) | orv in one VALU op.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t orv) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(orv));
    return r;
}

// Sum over one Q4_0 block of (q_e - 8) * x_e, e = 0..31.  Code byte j holds
// element j (low nibble) and element j + 16 (high nibble); dword i holds
// bytes 4i..4i+3.  A nibble at bits 0-3 of a 16-bit half, ORed under 0x6400,
// is the fp16 value 1024 + q; at bits 4-7 it is 1024 + 16q.  Subtracting 1032
// (or 1152) gives q - 8 (or 16 (q - 8)) exactly.  The high-nibble sum is
// therefore 16x too large and is scaled by 1/16 (exact) at the end.
__device__ __forceinline__ float dot_q4_0(const u32x4 c, const float (&x)[32]) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    const uint32_t kExp = 0x64006400u;
    const half2_t lo_off = {(_Float16)1032.0f, (_Float16)1032.0f};
    const half2_t hi_off = {(_Float16)1152.0f, (_Float16)1152.0f};
    float s_lo = 0.0f, s_hi = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t d = w[i];
        const uint32_t e = d >> 8;
        const half2_t t0 = as_half2(and_or(d, 0x000F000Fu, kExp)) - lo_off;  // elems 4i, 4i+2
        const half2_t t1 = as_half2(and_or(d, 0x00F000F0u, kExp)) - hi_off;  // 16+4i, 16+4i+2
        const half2_t t2 = as_half2(and_or(e, 0x000F000Fu, kExp)) - lo_off;  // 4i+1, 4i+3
        const half2_t t3 = as_half2(and_or(e, 0x00F000F0u, kExp)) - hi_off;  // 16+4i+1, 16+4i+3
        s_lo = __builtin_fmaf((float)t0.x, x[4 * i + 0], s_lo);
        s_lo = __builtin_fmaf((float)t2.x, x[4 * i + 1], s_lo);
        s_lo = __builtin_fmaf((float)t0.y, x[4 * i + 2], s_lo);
        s_lo = __builtin_fmaf((float)t2.y, x[4 * i + 3], s_lo);
        s_hi = __builtin_fmaf((float)t1.x, x[16 + 4 * i + 0], s_hi);
        s_hi = __builtin_fmaf((float)t3.x, x[16 + 4 * i + 1], s_hi);
        s_hi = __builtin_fmaf((float)t1.y, x[16 + 4 * i + 2], s_hi);
        s_hi = __builtin_fmaf((float)t3.y, x[16 + 4 * i + 3], s_hi);
    }
    return __builtin_fmaf(s_hi, 0.0625f, s_lo);
}

// Sum over 32 int8 codes (two 16-byte loads, element order) of c_e * x_e.
__device__ __forceinline__ float dot_i8(const u32x4 c0, const u32x4 c1, const float (&x)[32]) {
    const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t d = w[i];
        s0 = __builtin_fmaf((float)(int8_t)(d), x[4 * i + 0], s0);
        s1 = __builtin_fmaf((float)(int8_t)(d >> 8), x[4 * i + 1], s1);
        s0 = __builtin_fmaf((float)(int8_t)(d >> 16), x[4 * i + 2], s0);
        s1 = __builtin_fmaf((float)(int8_t)(d >> 24), x[4 * i + 3], s1);
    }
    return s0 + s1;
}

// Load the 32 activations of unit u (fp32 or fp16 -> fp32, exact) or zeros.
__device__ __forceinline__ void load_x_unit(const void* x, int xdt, int u, bool valid,
                                            float (&xr)[32]) {
    if (!valid) {
#pragma unroll
        for (int e = 0; e < 32; ++e) xr[e] = 0.0f;
        return;
    }
    if (xdt == kF32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + size_t(u) * 32);
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            const float4 t = p[v];
            xr[4 * v + 0] = t.x;
            xr[4 * v + 1] = t.y;
            xr[4 * v + 2] = t.z;
            xr[4 * v + 3] = t.w;
        }
    } else {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + size_t(u) * 32);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const uint4 t = p[v];
            const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const half2_t h = as_half2(w[q]);
                xr[8 * v + 2 * q + 0] = (float)h.x;
                xr[8 * v + 2 * q + 1] = (float)h.y;
            }
        }
    }
}

// Transposed butterfly over the TPW lanes of a team inside one wave: on entry
// every lane holds RPI partials (one per row); on exit the lane whose bits
// (TPW/2, TPW/4, ...) spell r holds the team's total for row r in v[0].
template <int RPI, int TPW>
__device__ __forceinline__ void team_reduce(float (&v)[RPI], int lt) {
    int n = RPI;
    int off = TPW / 2;
#pragma unroll
    for (int step = 0; (RPI >> step) > 1; ++step) {
        const int h = n / 2;
        const bool upper = (lt & off) != 0;
#pragma unroll
        for (int i = 0; i < RPI / 2; ++i) {
            if (i < h) {
                const float send = upper ? v[i] : v[i + h];
                const float keep = upper ? v[i + h] : v[i];
                v[i] = keep + __shfl_xor(send, off, 64);
            }
        }
        n = h;
        off >>= 1;
    }
#pragma unroll
    for (; off >= 1; off >>= 1) v[0] += __shfl_xor(v[0], off, 64);
}

// Row index held by lane lt after team_reduce.
template <int RPI, int TPW>
__device__ __forceinline__ int reduced_row(int lt) {
    int r = 0;
    int off = TPW / 2;
#pragma unroll
    for (int b = RPI / 2; b >= 1; b >>= 1) {
        if (lt & off) r += b;
        off >>= 1;
    }
    return r;
}

template <int FMT, int TP, int UPL>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(const GemvBatchArgs args) {
    constexpr int RPI = UPL == 1 ? 8 : (UPL == 2 ? 4 : 2);   // rows per team per iteration
    constexpr int TEAMS = kGemvThreads / TP;
    constexpr int ROWS = TEAMS * RPI;
    constexpr int CW = FMT == kQ4_0 ? 1 : 2;                  // 16-byte loads per unit
    constexpr int TPW = TP < 64 ? TP : 64;                    // team lanes inside one wave
    constexpr int WAVES_PER_TEAM = TP / TPW;

    __shared__ float red[kGemvThreads / 64][RPI];

    const int tid = threadIdx.x;
    const int team = tid / TP;
    const int lt = tid % TP;
    const int wl = tid % TPW;

    float xr[UPL][32];
    int cur = -1;
    const int total = args.prefix[args.count];

    for (int it = blockIdx.x; it < total; it += gridDim.x) {
        int di = 0;
        while (di + 1 < args.count && it >= args.prefix[di + 1]) ++di;
        const GemvDesc& D = args.d[di];
        const int nu = D.nu;
        const int nchunks = (nu + TP * UPL - 1) / (TP * UPL);
        const int row0 = (it - args.prefix[di]) * ROWS;

        float acc[RPI];
#pragma unroll
        for (int r = 0; r < RPI; ++r) acc[r] = 0.0f;

        for (int ch = 0; ch < nchunks; ++ch) {
            const int ubase = ch * TP * UPL;
            if (nchunks > 1 || di != cur) {
#pragma unroll
                for (int j = 0; j < UPL; ++j) {
                    const int u = ubase + lt + j * TP;
                    load_x_unit(D.x, D.xdt, u, u < nu, xr[j]);
                }
                cur = di;
            }
            u32x4 code[RPI][UPL][CW];
            float sc[RPI][UPL];
#pragma unroll
            for (int r = 0; r < RPI; ++r) {
                const int row = row0 + r * TEAMS + team;
#pragma unroll
                for (int j = 0; j < UPL; ++j) {
                    const int u = ubase + lt + j * TP;
                    const bool ok = row < D.N && u < nu;
                    const size_t unit = size_t(row) * size_t(nu) + size_t(u);
#pragma unroll
                    for (int c = 0; c < CW; ++c) code[r][j][c] = u32x4{0u, 0u, 0u, 0u};
                    sc[r][j] = 0.0f;
                    if (ok) {
                        const u32x4* cp = reinterpret_cast<const u32x4*>(D.codes + unit * (16 * CW));
#pragma unroll
                        for (int c = 0; c < CW; ++c) code[r][j][c] = __builtin_nontemporal_load(cp + c);
                        if (FMT == kI8B64) {
                            sc[r][j] = static_cast<const float*>(D.scales)[size_t(row) * size_t(nu / 2) + u / 2];
                        } else {
                            const _Float16 h = static_cast<const _Float16*>(D.scales)[unit];
                            sc[r][j] = (float)h;
                        }
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < RPI; ++r) {
#pragma unroll
                for (int j = 0; j < UPL; ++j) {
                    float s;
                    if (FMT == kQ4_0) s = dot_q4_0(code[r][j][0], xr[j]);
                    else s = dot_i8(code[r][j][0], code[r][j][CW - 1], xr[j]);
                    acc[r] = __builtin_fmaf(sc[r][j], s, acc[r]);
                }
            }
        }

        team_reduce<RPI, TPW>(acc, wl);
        const int rr = reduced_row<RPI, TPW>(wl);
        const bool owner = (wl % (TPW / RPI)) == 0;
        if (WAVES_PER_TEAM == 1) {
            const int row = row0 + rr * TEAMS + team;
            if (owner && row < D.N) D.y[row] = acc[0];
        } else {
            const int wave = tid / 64;
            if (owner) red[wave][rr] = acc[0];
            __syncthreads();
            if (tid < TEAMS * RPI) {
                const int tm = tid / RPI;
                const int r = tid % RPI;
                float s = 0.0f;
#pragma unroll
                for (int w = 0; w < WAVES_PER_TEAM; ++w) s += red[tm * WAVES_PER_TEAM + w][r];
                const int row = row0 + r * TEAMS + tm;
                if (row < D.N) D.y[row] = s;
            }
            __syncthreads();
        }
    }
}

struct Cand { int tp, upl; };
constexpr Cand kCands[] = {{16, 1}, {32, 1}, {64, 1}, {64, 2}, {64, 3},
                           {128, 2}, {128, 3}, {256, 1}, {256, 2}, {256, 3}};

template <int FMT>
hipError_t launch_fmt(const GemvConfig& cfg, const GemvBatchArgs& args, int grid, hipStream_t s) {
#define LQ_GEMV_CASE(TPv, UPLv)                                                         \
    if (cfg.tp == TPv && cfg.upl == UPLv) {                                             \
        hipLaunchKernelGGL((gemv_kernel<FMT, TPv, UPLv>), dim3(grid), dim3(kGemvThreads), \
                           0, s, args);                                                 \
        return hipGetLastError();                                                       \
    }
    LQ_GEMV_CASE(16, 1)
    LQ_GEMV_CASE(32, 1)
    LQ_GEMV_CASE(64, 1)
    LQ_GEMV_CASE(64, 2)
    LQ_GEMV_CASE(64, 3)
    LQ_GEMV_CASE(128, 2)
    LQ_GEMV_CASE(128, 3)
    LQ_GEMV_CASE(256, 1)
    LQ_GEMV_CASE(256, 2)
    LQ_GEMV_CASE(256, 3)
#undef LQ_GEMV_CASE
    return hipErrorInvalidValue;
}

}  // namespace

// Pick the team shape that wastes the fewest lane slots per row; a row longer
// than 768 units (K > 24576) is processed in chunks, reloading activations.
GemvConfig gemv_config(int nu) {
    int best = -1;
    long best_cost = 0;
    for (int i = 0; i < int(sizeof(kCands) / sizeof(kCands[0])); ++i) {
        const long slots = long(kCands[i].tp) * kCands[i].upl;
        const long chunks = (nu + slots - 1) / slots;
        // One chunk: fewest wasted lane slots.  Several chunks (activations
        // re-read per chunk): fewest chunks first.
        const long cost = chunks == 1 ? slots : (1L << 40) + chunks * (1L << 20) + slots * chunks;
        if (best < 0 || cost < best_cost ||
            (cost == best_cost && kCands[i].upl < kCands[best].upl)) {
            best = i;
            best_cost = cost;
        }
    }
    GemvConfig c;
    c.tp = kCands[best].tp;
    c.upl = kCands[best].upl;
    const int rpi = c.upl == 1 ? 8 : (c.upl == 2 ? 4 : 2);
    c.rows_per_iter = (kGemvThreads / c.tp) * rpi;
    return c;
}

hipError_t launch_gemv(int fmt, const GemvConfig& cfg, const GemvBatchArgs& args, int grid,
                       hipStream_t stream) {
    switch (fmt) {
        case kQ4_0: return launch_fmt<kQ4_0>(cfg, args, grid, stream);
        case kQ8_0: return launch_fmt<kQ8_0>(cfg, args, grid, stream);
        case kI8B64: return launch_fmt<kI8B64>(cfg, args, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lq
