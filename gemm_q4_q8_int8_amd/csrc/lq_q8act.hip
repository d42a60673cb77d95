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
//     load; each adds its own dot products, so the vector work grows with
//     the token count.
//   * gemv_q8act_mfma_kernel (more tokens, q8act_mfma_from): the same exact
//     block sums on the integer matrix cores, below.
#include "lq_frag.h"
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

// N consecutive wave-uniform dwords (N = 1, 2, 4, 8 or a multiple of 16) as
// the widest scalar loads (dword alignment is all a scalar load needs).
template <int N>
__device__ __forceinline__ void sload(ci32_p p, int32_t (&o)[N]) {
    typedef int32_t v16 __attribute__((ext_vector_type(16), aligned(4)));
    typedef int32_t v8 __attribute__((ext_vector_type(8), aligned(4)));
    typedef int32_t v4 __attribute__((ext_vector_type(4), aligned(4)));
    typedef int32_t v2 __attribute__((ext_vector_type(2), aligned(4)));
    if constexpr (N % 16 == 0) {
#pragma unroll
        for (int i = 0; i < N / 16; ++i) {
            const v16 v = *reinterpret_cast<const __attribute__((address_space(4))) v16*>(p + 16 * i);
#pragma unroll
            for (int k = 0; k < 16; ++k) o[16 * i + k] = v[k];
        }
    } else if constexpr (N == 8) {
        const v8 v = *reinterpret_cast<const __attribute__((address_space(4))) v8*>(p);
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = v[k];
    } else if constexpr (N == 4) {
        const v4 v = *reinterpret_cast<const __attribute__((address_space(4))) v4*>(p);
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = v[k];
    } else if constexpr (N == 2) {
        const v2 v = *reinterpret_cast<const __attribute__((address_space(4))) v2*>(p);
        o[0] = v[0];
        o[1] = v[1];
    } else {
        static_assert(N == 1, "dword count");
        o[0] = p[0];
    }
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
        tile = int(uint32_t(local) / uint32_t(S));
        slice = local - tile * S;
        slice_units(nu, S, slice, sa, sb);
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
        auto load_scale = [&](int k) {
            const uint32_t so = uint32_t(min(u + k, ub - 1)) * s_unit + s_lane;
            if constexpr (SB == 2) sw[k] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(sbase + so));
            else sw[k] = *reinterpret_cast<const uint32_t*>(sbase + so);
        };
        auto load_codes = [&](int k) {
            const uint32_t co = uint32_t(min(u + k, ub - 1)) * c_unit + c_lane;
#pragma unroll
            for (int p = 0; p < P; ++p)
                cw[k][p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(cbase + co + uint32_t(p) * c_part));
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
        __builtin_amdgcn_sched_barrier(0);
        // Q4_0: code dword i's low nibbles are elements 4i .. 4i + 3 of the
        // block, its high nibbles 16 + 4i .., both as the stored values q + 8
        // (0 .. 15); the int8 formats: code part 2 xb + h holds elements
        // 16 h .. 16 h + 15 of the unit's block xb.
        auto codes_of = [&](int k, int xb, uint32_t (&c)[8]) {
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
        };
        if (u + UNR <= ub) {
            // A whole batch: each token's activation codes, scales and code
            // sums of the batch's UNR * XB consecutive blocks in a few wide
            // scalar loads (one load of each per block and token made this
            // kernel bound by the CU's scalar unit: 402 scalar instructions
            // per wave at four tokens).
            constexpr int NB = UNR * XB;
            uint32_t c[NB][8];
#pragma unroll
            for (int k = 0; k < UNR; ++k)
#pragma unroll
                for (int xb = 0; xb < XB; ++xb) codes_of(k, xb, c[k * XB + xb]);
            float ws[UNR];
#pragma unroll
            for (int k = 0; k < UNR; ++k) {
                if constexpr (fp32_scale(FMT)) ws[k] = __uint_as_float(sw[k]);
                else ws[k] = (float)__builtin_bit_cast(_Float16, uint16_t(sw[k]));
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const size_t b0 = size_t(t) * size_t(nb) + size_t(u) * XB;
                int32_t xq[NB * 8], xs[NB], xsum[NB];
                sload<NB * 8>((ci32_p)(a.q) + b0 * 8, xq);
                sload<NB>((ci32_p)(a.s) + b0, xs);
                if constexpr (FMT == kQ4_0) sload<NB>((ci32_p)(a.sum) + b0, xsum);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    int I = FMT == kQ4_0 ? -8 * xsum[b] : 0;
#pragma unroll
                    for (int i = 0; i < 8; ++i) I = __builtin_amdgcn_sdot4(int(c[b][i]), xq[8 * b + i], I, false);
                    acc[t] = __builtin_fmaf(ws[b / XB] * __int_as_float(xs[b]), float(I), acc[t]);
                }
            }
            continue;
        }
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


// ------------------------------------------------ matrix-core variant ----
// The same product for several tokens on the integer matrix cores: one
// v_mfma_i32_16x16x32_i8 per (16 weight rows, one 32-element block), A = the
// 16-token activation code fragment, B = the weight codes as int8 (Q4_0: the
// stored nibbles q + 8, with the accumulator started at -8 x the block's code
// sum), so the block sums are the same exact integers as above.  Layout as
// the fp16 multi-token GEMV's: lane (r, g) (r = lane % 16, g = lane / 16)
// loads tile row 4r + g; four cross-row swaps give lane (r, j) code dword j
// of rows 4r .. 4r+3; the output lane (r, j) holds tokens 4j .. 4j+3 of
// rows 4r .. 4r+3.  k order inside a block: Q4_0 lane group j takes elements
// 4j .. 4j+3 and 16+4j .. 16+4j+3 (the low and high nibbles of code dword
// j), the int8 formats elements 8j .. 8j+7.
//
// Each wave stages its batch's activation codes (token rows of the batch's
// K range), scales and code sums (block-major, 16 tokens per block) in its
// own LDS area with global_load_lds; reading them straight from memory
// would make every load touch 16 token rows.
template <int FMT, int UNR>
struct Q8Stage {
    static constexpr int E = unit_elems(FMT);
    static constexpr int XB = E / 32;                    // activation blocks per unit
    static constexpr int CPU = E / 16;                   // 16-byte chunks of codes per unit and token
    static constexpr int P16 = UNR * CPU + 1;            // code row pitch in chunks (odd: no bank conflicts)
    static constexpr int kQBytes = (16 * P16 + 63) / 64 * 1024;
    static constexpr int kSDwords = (UNR * XB * 16 + 63) / 64 * 64;
    static constexpr int kSums = FMT == kQ4_0 ? 1 : 0;   // code sums staged (Q4_0 only)
    static constexpr int kBytes = kQBytes + (1 + kSums) * kSDwords * 4;
};

template <int FMT>
struct Q8Unit {
    u32x4 c[unit_parts(FMT)];   // codes of tile row 4r + g
    uint32_t s[4];              // raw scales of rows 4r .. 4r+3 (as the multi-token GEMV loads them)
};

template <int FMT, bool FULL>
__device__ __forceinline__ float q8_scale(const Q8Unit<FMT>& b, int m) {
    if constexpr (scale_bytes(FMT) == 4) {
        return __uint_as_float(b.s[m]);
    } else {
        const uint32_t v = FULL ? b.s[m >> 1] : b.s[m];
        const uint16_t h = uint16_t(FULL && (m & 1) ? v >> 16 : v);
        return (float)__builtin_bit_cast(_Float16, h);
    }
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct Q8Wave {
    const uint8_t* cbase;   // code plane of the tile
    const uint8_t* sbase;   // scale plane of the tile
    uint8_t* xs;            // this wave's staging area
    uint32_t c_lane, c_unit, c_part, s_unit;
    uint32_t s_row[4];
    uint32_t q_row;         // byte offset of this lane's token row in the staged codes
    int ua, ub, nb, K;
};

template <int FMT, int UNR, bool FULL>
__device__ __forceinline__ void q8_accumulate(const Q8ActArgs& a, const Q8Wave& L, f32x4 (&acc)[4]) {
    using QS = Q8Stage<FMT, UNR>;
    constexpr int P = unit_parts(FMT);
    constexpr int SB = scale_bytes(FMT);
    constexpr int E = QS::E;
    constexpr int XB = QS::XB;
    const int lane = int(threadIdx.x) & 63;
    const int g = lane >> 4;
    const int M = a.M;
    uint8_t* const xq = L.xs;
    uint8_t* const xsc = L.xs + QS::kQBytes;
    uint8_t* const xsm = xsc + QS::kSDwords * 4;
    for (int u = L.ua; u < L.ub; u += UNR) {
        // Codes: lane l of copy i fills chunk q = 64 i + l: token row
        // t = q / P16 (token min(t, M - 1)), chunk kc of the row: unit
        // min(u + kc / CPU, ub - 1), its chunk kc % CPU.  Scales and sums:
        // dword p = 64 i + l is block slot p / 16 (unit (p / 16) / XB,
        // sub-block (p / 16) % XB) of token p % 16.  Pads, slack and rows
        // past M re-read valid data nobody uses.
        const int ni = (M * QS::P16 + 63) / 64;
        for (int i = 0; i < ni; ++i) {
            const int q = 64 * i + lane;
            const int t = min(q / QS::P16, M - 1);
            const int kc = min(q % QS::P16, UNR * QS::CPU - 1);
            const int uk = min(u + kc / QS::CPU, L.ub - 1);
            const size_t off = size_t(t) * size_t(L.K) + size_t(uk) * E + size_t(kc % QS::CPU) * 16;
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(a.q + off),
                                             (__attribute__((address_space(3))) void*)(xq + 1024 * i), 16, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < QS::kSDwords / 64; ++i) {
            const int p = 64 * i + lane;
            const int bs = p >> 4;
            const int t = min(p & 15, M - 1);
            const int uk = min(u + bs / XB, L.ub - 1);
            const size_t idx = size_t(t) * size_t(L.nb) + size_t(uk) * XB + size_t(bs % XB);
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(a.s + idx),
                                             (__attribute__((address_space(3))) void*)(xsc + 256 * i), 4, 0, 0);
            if constexpr (QS::kSums)
                __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(a.sum + idx),
                                                 (__attribute__((address_space(3))) void*)(xsm + 256 * i), 4, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        Q8Unit<FMT> b[UNR];
        auto load_scale = [&](int k) {
            const uint32_t uu = uint32_t(min(u + k, L.ub - 1));
            const uint8_t* sp = L.sbase + uu * L.s_unit;
            if constexpr (FULL && SB == 2) {
                const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(sp + L.s_row[0]));
                b[k].s[0] = v.x;
                b[k].s[1] = v.y;
            } else if constexpr (FULL) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(sp + L.s_row[0]);
                b[k].s[0] = v.x;
                b[k].s[1] = v.y;
                b[k].s[2] = v.z;
                b[k].s[3] = v.w;
            } else {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    if constexpr (SB == 2)
                        b[k].s[m] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(sp + L.s_row[m]));
                    else b[k].s[m] = *reinterpret_cast<const uint32_t*>(sp + L.s_row[m]);
                }
            }
        };
        auto load_codes = [&](int k) {
            const uint32_t uu = uint32_t(min(u + k, L.ub - 1));
            const uint32_t co = uu * L.c_unit + L.c_lane;
#pragma unroll
            for (int p = 0; p < P; ++p)
                b[k].c[p] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4*>(L.cbase + co + uint32_t(p) * L.c_part));
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
        // The copies into LDS were issued before the batch's code and scale
        // loads, and the vector-memory counter is in order: they have landed
        // once at most those loads are outstanding.
        __builtin_amdgcn_sched_barrier(0);
        constexpr int kBatchLoads = UNR * (P + (FULL ? 1 : 4));
        static_assert(kBatchLoads <= 63, "vmcnt range");
        __builtin_amdgcn_s_waitcnt((kBatchLoads & 15) | (0x7 << 4) | (0xF << 8) | ((kBatchLoads >> 4) << 14));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < UNR; ++k) {
            if (u + k >= L.ub) continue;
            u32x4 t[P];
            if constexpr (FMT == kQ4_0) {
                t[0] = frag::xpose(b[k].c[0]);
            } else {
#pragma unroll
                for (int ks = 0; ks < XB; ++ks) {
                    const u32x4 p0 = b[k].c[2 * ks], p1 = b[k].c[2 * ks + 1];
                    t[2 * ks] = frag::xpose(u32x4{p0.x, p0.z, p1.x, p1.z});
                    t[2 * ks + 1] = frag::xpose(u32x4{p0.y, p0.w, p1.y, p1.w});
                }
            }
#pragma unroll
            for (int xb = 0; xb < XB; ++xb) {
                const uint8_t* qp = xq + L.q_row + (k * QS::CPU) * 16 + 32 * xb;
                uint64_t A;
                if constexpr (FMT == kQ4_0) {
                    const uint32_t lo = *reinterpret_cast<const uint32_t*>(qp + 4 * g);
                    const uint32_t hi = *reinterpret_cast<const uint32_t*>(qp + 16 + 4 * g);
                    A = uint64_t(lo) | (uint64_t(hi) << 32);
                } else {
                    A = *reinterpret_cast<const uint64_t*>(qp + 8 * g);
                }
                const int bs = k * XB + xb;
                const f32x4 sx = *reinterpret_cast<const f32x4*>(xsc + (bs * 16 + 4 * g) * 4);
                i32x4 c0 = {0, 0, 0, 0};
                if constexpr (FMT == kQ4_0) c0 = *reinterpret_cast<const i32x4*>(xsm + (bs * 16 + 4 * g) * 4) * -8;
                // The four row groups' block sums first, then their scaling
                // (a use right behind the MFMA would wait for its result).
                i32x4 I[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    uint64_t B;
                    if constexpr (FMT == kQ4_0)
                        B = uint64_t(t[0][m] & 0x0F0F0F0Fu) | (uint64_t((t[0][m] >> 4) & 0x0F0F0F0Fu) << 32);
                    else B = uint64_t(t[2 * xb][m]) | (uint64_t(t[2 * xb + 1][m]) << 32);
                    I[m] = __builtin_amdgcn_mfma_i32_16x16x32_i8(long(A), long(B), c0, 0, 0, 0);
                }
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float ws = q8_scale<FMT, FULL>(b[k], m);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[m][i] = __builtin_fmaf(ws * sx[i], float(I[m][i]), acc[m][i]);
                }
            }
        }
    }
}

template <int FMT, int UNR>
__global__ __launch_bounds__(256) void gemv_q8act_mfma_kernel(const Q8ActArgs a) {
    constexpr int UB = unit_bytes(FMT);
    constexpr int SB = scale_bytes(FMT);
    using QS = Q8Stage<FMT, UNR>;
    constexpr int kStageBytes = 4 * QS::kBytes;
    constexpr int kRedBytes = 4 * 16 * 64 * 4;
    __shared__ __attribute__((aligned(16))) uint8_t smem[kStageBytes > kRedBytes ? kStageBytes : kRedBytes];
    __shared__ uint32_t last;
    auto red = reinterpret_cast<float (*)[16][64]>(smem);

    const int N = a.N, nu = a.nu, S = a.S, M = a.M;
    const int local = int(blockIdx.x);
    const int tile = int(uint32_t(local) / uint32_t(S));
    const int slice = local - tile * S;
    const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    const int lane = int(threadIdx.x) & 63;
    const int r = lane & 15, g = lane >> 4;
    const int nr = min(kTileRows, N - tile * kTileRows);
    const bool full = nr == kTileRows;
    int sa, sb;
    slice_units(nu, S, slice, sa, sb);

    const size_t first = size_t(tile) * kTileRows * size_t(nu);
    Q8Wave L;
    L.cbase = a.codes + first * UB;
    L.sbase = a.scales + first * SB;
    L.xs = smem + w * QS::kBytes;
    // Rows past the end of a partial tile are re-read from the last row and
    // never stored; so are tokens past M.
    L.c_lane = uint32_t(min(4 * r + g, nr - 1)) * 16u;
    L.c_unit = uint32_t(nr) * UB;
    L.c_part = uint32_t(nr) * 16u;
    L.s_unit = uint32_t(nr) * SB;
#pragma unroll
    for (int m = 0; m < 4; ++m) L.s_row[m] = uint32_t(min(4 * r + m, nr - 1)) * SB;
    L.q_row = uint32_t(min(r, M - 1)) * uint32_t(QS::P16) * 16u;
    L.ua = __builtin_amdgcn_readfirstlane(sa + (sb - sa) * w / 4);
    L.ub = __builtin_amdgcn_readfirstlane(sa + (sb - sa) * (w + 1) / 4);
    L.nb = nu * QS::XB;
    L.K = nu * QS::E;

    f32x4 acc[4] = {};
    if (full) q8_accumulate<FMT, UNR, true>(a, L, acc);
    else q8_accumulate<FMT, UNR, false>(a, L, acc);

    // Sum the four waves' K quarters (the staging areas are free once every
    // wave is past its loop); wave w then owns token 4g + w of rows 4r .. 4r+3.
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[w][4 * m + i][lane] = acc[m][i];
    __syncthreads();
    float v[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
        v[m] = (red[0][4 * m + w][lane] + red[1][4 * m + w][lane]) +
               (red[2][4 * m + w][lane] + red[3][4 * m + w][lane]);
    const int token = 4 * g + w;
    const size_t row0 = size_t(tile) * kTileRows + size_t(4 * r);
    if (S == 1) {
        if (token < M) {
            float* yp = a.y + size_t(token) * size_t(N) + row0;
#pragma unroll
            for (int m = 0; m < 4; ++m)
                if (4 * r + m < nr) yp[m] = v[m];
        }
        return;
    }
    // Split K: the hand-off of lq_splitk.h (slice j of token t at rows
    // (j M + t) pitch of the partials).
    const size_t pitch = size_t(a.tiles) * kTileRows;
    const size_t spitch = pitch * size_t(M);
    if (token < M) {
        float* pp = a.part + size_t(slice) * spitch + size_t(token) * pitch + row0;
#pragma unroll
        for (int m = 0; m < 4; ++m) splitk_put(pp + m, v[m]);
    }
    splitk_publish();
    __syncthreads();
    if (threadIdx.x == 0) last = splitk_arrive(&a.cnt[tile], a.tag, S) ? 1u : 0u;
    __syncthreads();
    if (!last) return;
    if (token < M) {
        const float* pp = a.part + size_t(token) * pitch + row0;
        float* yp = a.y + size_t(token) * size_t(N) + row0;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float t = sum_slices(pp + m, spitch, S);
            if (4 * r + m < nr) yp[m] = t;
        }
    }
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

hipError_t launch_gemv_q8act_mfma(int fmt, const Q8ActArgs& a, hipStream_t stream) {
    const dim3 grid(unsigned(int64_t(a.tiles) * a.S)), block(256u);
    // (Q4_0 batches of 7 units, one per wave on the 151936 x 896 LM head,
    // measured slower than batches of 4 and 3: 26.5 against 24.3 us at
    // M = 16, at 112 instead of 86 registers.)
    switch (fmt) {
        case kQ4_0: hipLaunchKernelGGL((gemv_q8act_mfma_kernel<kQ4_0, 4>), grid, block, 0, stream, a); break;
        case kQ8_0: hipLaunchKernelGGL((gemv_q8act_mfma_kernel<kQ8_0, 2>), grid, block, 0, stream, a); break;
        case kI8B64: hipLaunchKernelGGL((gemv_q8act_mfma_kernel<kI8B64, 2>), grid, block, 0, stream, a); break;
        case kI8B32: hipLaunchKernelGGL((gemv_q8act_mfma_kernel<kI8B32, 2>), grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Token counts the vector kernel is built for: those below q8act_mfma_from.
template <int FMT>
constexpr auto vector_token_counts() {
    constexpr int n = q8act_mfma_from(FMT) - 1 < kQ8ActMaxTokens ? q8act_mfma_from(FMT) - 1 : kQ8ActMaxTokens;
    static_assert(n >= 1, "the vector kernel takes at least one token count");
    return std::make_integer_sequence<int, n>{};
}

hipError_t launch_gemv_q8act(int fmt, const Q8ActArgs& a, int waves, hipStream_t stream) {
    if (waves != 4 && waves != 16) return hipErrorInvalidValue;
    switch (fmt) {
        case kQ4_0: return launch_fmt<kQ4_0>(a, waves, stream, vector_token_counts<kQ4_0>());
        case kQ8_0: return launch_fmt<kQ8_0>(a, waves, stream, vector_token_counts<kQ8_0>());
        case kI8B64: return launch_fmt<kI8B64>(a, waves, stream, vector_token_counts<kI8B64>());
        case kI8B32: return launch_fmt<kI8B32>(a, waves, stream, vector_token_counts<kI8B32>());
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lq
