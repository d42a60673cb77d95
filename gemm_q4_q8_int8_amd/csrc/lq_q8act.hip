// Activation-quantized integer-dot GEMV: per-matmul int8 quantization of the
// activations, then int8 dot products with the weight codes.
//
// The "oxinfer" page's decode kernels quantize each matmul's activations and
// take int8 dot products of them with the quantized weights, four blocks at a
// time, with multi-token variants for verifying drafted tokens ("How it
// works", quant.rs); at Q4 those multi-token kernels are instruction bound
// ("Speculative decoding").  Here:
//   * quantize_act_kernel: one thread per 32-element block of a token row:
//     s = max|x| / 127, q = clamp(rint(x / s), +-127) (fp32 steps, the page's
//     Q8 rule), and the block's code sum (Q4_0 codes are stored as q + 8, so
//     sum_k (q_w - 8) q_x = sum_k q_w q_x - 8 sum_k q_x).
//   * gemv_q8act_kernel: the GEMV's tiled row-per-lane layout (lane r owns
//     row r of a 64-row tile, every code load one coalesced 1 KB run); the
//     quantized activations are wave-uniform and come from the scalar cache.
//     Each 32-element block is 8 v_dot4 (signed bytes, int32 accumulate):
//     Q4_0's low nibbles of code dword i are elements 4i .. 4i + 3 and its
//     high nibbles 16 + 4i .. 16 + 4i + 3, so both dot the activations in
//     their natural order.  The exact block sum I becomes fp32 (|I| < 2^24)
//     and is scaled once: acc += fl(ws * s) * I.  Tokens share every code
//     load; each adds its own dot products.
#include "lq_splitk.h"

#include <utility>

namespace lq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(4))) int32_t* ci32_p;
typedef const __attribute__((address_space(4))) float* cf32_p;

constexpr int kActThreads = 256;

__device__ __forceinline__ int round_clamp127(float v) { return int(fminf(fmaxf(rintf(v), -127.0f), 127.0f)); }

template <int XDT>
__global__ __launch_bounds__(kActThreads) void quantize_act_kernel(const void* __restrict__ X,
                                                                   int8_t* __restrict__ q, float* __restrict__ s,
                                                                   int32_t* __restrict__ sum, int64_t blocks) {
    const int64_t b = int64_t(blockIdx.x) * kActThreads + threadIdx.x;
    if (b >= blocks) return;
    float x[32];
    if constexpr (XDT == kF32) {
        const float* p = static_cast<const float*>(X) + b * 32;
#pragma unroll
        for (int e = 0; e < 32; ++e) x[e] = p[e];
    } else {
        const _Float16* p = static_cast<const _Float16*>(X) + b * 32;
#pragma unroll
        for (int e = 0; e < 32; ++e) x[e] = float(p[e]);
    }
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) a = fabsf(x[e]) > a ? fabsf(x[e]) : a;
    const float sc = a / 127.0f;
    int32_t t = 0;
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t v = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int c = sc == 0.0f ? 0 : round_clamp127(x[4 * i + k] / sc);
            t += c;
            v |= uint32_t(uint8_t(int8_t(c))) << (8 * k);
        }
        w[i] = v;
    }
    u32x4* qo = reinterpret_cast<u32x4*>(q + b * 32);
    qo[0] = u32x4{w[0], w[1], w[2], w[3]};
    qo[1] = u32x4{w[4], w[5], w[6], w[7]};
    s[b] = sc;
    sum[b] = t;
}

// Integer dot product of one block, added to I: code dwords c[0..7] (signed
// bytes; for Q4_0 the nibbles of the 4 code dwords, below) with activation
// dwords x[0..7].
template <int FMT>
__device__ __forceinline__ int block_dot(const uint32_t (&c)[8], ci32_p x, int I) {
#pragma unroll
    for (int i = 0; i < 8; ++i) I = __builtin_amdgcn_sdot4(int(c[i]), x[i], I, false);
    return I;
}

// W waves per workgroup (4, or 16 when K is split several ways: four of the
// slices then meet in LDS instead of through the workspace) split a tile's K
// slice; UNR units per load batch; MT tokens (one instance per token count,
// so that the token loop is straight code whose activation loads the
// compiler can issue ahead).
template <int FMT, int MT, int UNR, int W>
__global__ __launch_bounds__(64 * W) void gemv_q8act_kernel(const Q8ActArgs a) {
    constexpr int P = unit_parts(FMT);
    constexpr int UB = unit_bytes(FMT);
    constexpr int SB = scale_bytes(FMT);
    constexpr int XB = unit_elems(FMT) / 32;   // activation blocks per unit
    __shared__ float red[MT][W][kTileRows];

    const int N = a.N, nu = a.nu, S = a.S;
    const int nb = nu * XB;                    // activation blocks per token row
    const int local = blockIdx.x;
    int tile = local, slice = 0, sa = 0, sb = nu;
    if (S > 1) {
        tile = local / S;
        slice = local - tile * S;
        sa = int(int64_t(nu) * slice / S);
        sb = int(int64_t(nu) * (slice + 1) / S);
    }
    const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    const int r = int(threadIdx.x) & 63;
    const int nr = min(kTileRows, N - tile * kTileRows);
    const int rc = min(r, nr - 1);
    const int ua = __builtin_amdgcn_readfirstlane(sa + (sb - sa) * w / W);
    const int ub = __builtin_amdgcn_readfirstlane(sa + (sb - sa) * (w + 1) / W);

    const size_t first = size_t(tile) * kTileRows * size_t(nu);
    const uint8_t* cbase = a.codes + first * UB;
    const uint8_t* sbase = a.scales + first * SB;
    const uint32_t c_lane = uint32_t(rc) * 16u;
    const uint32_t c_unit = uint32_t(nr) * UB;
    const uint32_t c_part = uint32_t(nr) * 16u;
    const uint32_t s_lane = uint32_t(rc) * SB;
    const uint32_t s_unit = uint32_t(nr) * SB;

    float acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = 0.0f;
    for (int u = ua; u < ub; u += UNR) {
        u32x4 cw[UNR][P];
        uint32_t sw[UNR];
#pragma unroll
        for (int k = 0; k < UNR; ++k) {
            const uint32_t uu = uint32_t(min(u + k, ub - 1));
            const uint32_t co = uu * c_unit + c_lane;
#pragma unroll
            for (int p = 0; p < P; ++p)
                cw[k][p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(cbase + co + uint32_t(p) * c_part));
            const uint32_t so = uu * s_unit + s_lane;
            if constexpr (SB == 2) sw[k] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(sbase + so));
            else sw[k] = *reinterpret_cast<const uint32_t*>(sbase + so);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < UNR; ++k) {
            if (u + k >= ub) break;   // uniform
            const int uu = u + k;
            float ws;
            if constexpr (fp32_scale(FMT)) ws = __uint_as_float(sw[k]);
            else ws = (float)__builtin_bit_cast(_Float16, uint16_t(sw[k]));
#pragma unroll
            for (int xb = 0; xb < XB; ++xb) {
                // c[i] pairs with activation dword i (elements 4i .. 4i + 3).
                // Q4_0: code dword i's low nibbles are elements 4i .. 4i + 3,
                // its high nibbles 16 + 4i .. 16 + 4i + 3, both as the stored
                // values q + 8 (0 .. 15, nonnegative bytes); the block's
                // activation code sum times 8 starts the dot product.
                uint32_t c[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (FMT == kQ4_0) {
                        c[i] = cw[k][0][i] & 0x0F0F0F0Fu;
                        c[4 + i] = (cw[k][0][i] >> 4) & 0x0F0F0F0Fu;
                    } else {
                        c[i] = cw[k][2 * xb][i];
                        c[4 + i] = cw[k][2 * xb + 1][i];
                    }
                }
                const size_t bx = size_t(uu) * XB + xb;
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const size_t xi = size_t(t) * size_t(nb) + bx;
                    const int I0 = FMT == kQ4_0 ? -8 * ((ci32_p)(a.sum))[xi] : 0;
                    const int I = block_dot<FMT>(c, (ci32_p)(a.q) + xi * 8, I0);
                    acc[t] = __builtin_fmaf(ws * ((cf32_p)(a.s))[xi], float(I), acc[t]);
                }
            }
        }
    }

#pragma unroll
    for (int t = 0; t < MT; ++t) red[t][w][r] = acc[t];
    __syncthreads();
    if (w != 0) return;
    float v[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        float p[W];
#pragma unroll
        for (int j = 0; j < W; ++j) p[j] = red[t][j][r];
#pragma unroll
        for (int h = 1; h < W; h *= 2)
#pragma unroll
            for (int j = 0; j < W; j += 2 * h) p[j] += p[j + h];
        v[t] = p[0];
    }
    const size_t row = size_t(tile) * kTileRows + size_t(r);
    if (S == 1) {
        if (r < nr) {
#pragma unroll
            for (int t = 0; t < MT; ++t) a.y[size_t(t) * N + row] = v[t];
        }
        return;
    }
    // Split K: the hand-off of lq_splitk.h (slice j of token t at rows
    // (j MT + t) pitch of the partials).
    const size_t pitch = size_t(a.tiles) * kTileRows;
#pragma unroll
    for (int t = 0; t < MT; ++t) splitk_put(&a.part[(size_t(slice) * MT + t) * pitch + row], v[t]);
    splitk_publish();
    uint32_t last = 0;
    if (r == 0) last = splitk_arrive(&a.cnt[tile], a.tag, S) ? 1u : 0u;
    last = __builtin_amdgcn_readfirstlane(last);
    if (!last) return;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const float y = sum_slices(a.part + size_t(t) * pitch + row, MT * pitch, S);
        if (r < nr) a.y[size_t(t) * N + row] = y;
    }
}

template <int FMT, int MT>
hipError_t launch_fmt_mt(const Q8ActArgs& a, int waves, hipStream_t stream) {
    constexpr int UNR = FMT == kQ4_0 ? 4 : (FMT == kI8B64 ? 1 : 2);
    const dim3 grid(unsigned(int64_t(a.tiles) * a.S));
    if (waves == 16) hipLaunchKernelGGL((gemv_q8act_kernel<FMT, MT, UNR, 16>), grid, dim3(1024u), 0, stream, a);
    else hipLaunchKernelGGL((gemv_q8act_kernel<FMT, MT, UNR, 4>), grid, dim3(256u), 0, stream, a);
    return hipGetLastError();
}

template <int FMT, int... Ms>
hipError_t launch_fmt(const Q8ActArgs& a, int waves, hipStream_t stream, std::integer_sequence<int, Ms...>) {
    using Fn = hipError_t (*)(const Q8ActArgs&, int, hipStream_t);
    static constexpr Fn table[] = {&launch_fmt_mt<FMT, Ms + 1>...};
    if (a.M < 1 || a.M > int(sizeof...(Ms))) return hipErrorInvalidValue;
    return table[a.M - 1](a, waves, stream);
}

}  // namespace

hipError_t launch_quantize_act(int xdt, const void* X, int64_t M, int64_t K, int8_t* q, float* s, int32_t* sum,
                               hipStream_t stream) {
    const int64_t blocks = M * (K / 32);
    const dim3 grid(unsigned((blocks + kActThreads - 1) / kActThreads)), block(kActThreads);
    if (xdt == kF32) hipLaunchKernelGGL((quantize_act_kernel<kF32>), grid, block, 0, stream, X, q, s, sum, blocks);
    else if (xdt == kF16) hipLaunchKernelGGL((quantize_act_kernel<kF16>), grid, block, 0, stream, X, q, s, sum, blocks);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_gemv_q8act(int fmt, const Q8ActArgs& a, int waves, hipStream_t stream) {
    if (waves != 4 && waves != 16) return hipErrorInvalidValue;
    const auto ms = std::make_integer_sequence<int, kQ8ActMaxTokens>{};
    switch (fmt) {
        case kQ4_0: return launch_fmt<kQ4_0>(a, waves, stream, ms);
        case kQ8_0: return launch_fmt<kQ8_0>(a, waves, stream, ms);
        case kI8B64: return launch_fmt<kI8B64>(a, waves, stream, ms);
        case kI8B32: return launch_fmt<kI8B32>(a, waves, stream, ms);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lq
