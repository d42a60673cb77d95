// Multi-token GEMV: Y[t, n] = sum_k w[n, k] X[t, k] for t < M <= 16 tokens,
// fp16 activations, weights in the tiled packed layout (Q4_0 / Q8_0 / int8
// block-64).  This is the decode step of a few tokens at once, as when a
// drafted run of tokens is verified in one pass ("oxinfer" page, "Speculative
// decoding"; "How it works", the multi-token variants of the decode kernels).
//
// The weights are still read once, so the step stays bound by HBM bandwidth
// for any M <= 16, while the arithmetic grows M-fold.  Per-lane FMAs would
// make it instruction-bound (the page observes exactly that for its Q4
// multi-token kernels), so the products run on the matrix cores:
//   * One v_mfma_f32_16x16x32_f16 per (16 rows, one 32-element block): A is
//     the 16 x 32 activation fragment (row = token), B the 32 x 16 weight
//     fragment (column = weight row) holding the EXACT integer codes (q - 8
//     or c) as fp16.  Products are exact and the block sum is fp32, so the
//     block scale is applied afterwards by an fp32 FMA: no weight is rounded
//     to fp16, and the result meets the GEMV accuracy bound, not the looser
//     one of the fp16-tile GEMM.
//   * A workgroup of 4 waves takes one 64-row tile and splits its units four
//     ways (and K across workgroups when the matrix has few tiles), like the
//     single-token GEMV, with the same split-K workspace hand-off.
//   * Lane (r, g) (r = lane % 16, g = lane / 16) loads tile row 4r + g of a
//     unit with one 16-byte load: the wave's load is the unit's contiguous
//     1 KB run.  Four cross-row swaps (v_permlane32_swap, v_permlane16_swap)
//     transpose the 4 x 4 dwords of lanes r, r+16, r+32, r+48, after which
//     lane (r, j) holds dword j of rows 4r, 4r+1, 4r+2, 4r+3: the B fragment
//     of row group m (weight rows 4r + m as column r) for k-set j.
//   * The MFMA output lane (r, j) then holds tokens 4j..4j+3 of weight rows
//     4r + m, so the scales it needs are the four consecutive ones of rows
//     4r..4r+3: one 8- or 16-byte load per unit.
//   * The k order inside a block is free as long as A and B agree.  Q4_0:
//     lane group j takes elements 4j..4j+3 and 16+4j..16+4j+3, exactly the
//     low and high nibbles of code dword j; those activations are staged in
//     LDS per batch of units (XStage below).  int8: lane group j takes
//     elements 8j..8j+7 (the two 16-byte parts of a 32-element step are
//     transposed as double dwords), so its activations are one 16-byte
//     load.
#include "lq_frag.h"
#include "lq_splitk.h"

namespace lq {
namespace {

using namespace frag;

// 32-element steps (MFMAs per row group) in one unit.
template <int FMT>
constexpr int steps_of() { return FMT == kI8B64 ? 2 : 1; }

template <int FMT>
struct MUnit {
    static constexpr int P = unit_parts(FMT);
    static constexpr int KS = steps_of<FMT>();
    u32x4 c[P];          // codes of tile row 4r + g (this lane's load)
    u32x2 xl[KS], xh[KS];  // activations of this lane's token and k-set
    // Raw scales of rows 4r .. 4r+3, as loaded: fp32 in s[0..3]; fp16 as two
    // packed dwords s[0..1] (full tile) or one per dword (partial tile).
    // Unpacking waits until use so that no ALU op follows a load directly
    // (it would make the load phase wait for its data).
    uint32_t s[4];
};

// fp32 scale of row 4r + m.
template <int FMT, bool FULL>
__device__ __forceinline__ float scale_of(const MUnit<FMT>& b, int m) {
    if constexpr (scale_bytes(FMT) == 4) {
        return __uint_as_float(b.s[m]);
    } else {
        const uint32_t v = FULL ? b.s[m >> 1] : b.s[m];
        const uint16_t h = uint16_t(FULL && (m & 1) ? v >> 16 : v);
        return (float)__builtin_bit_cast(_Float16, h);
    }
}

// Where one wave reads: tile bases, per-lane offsets and its unit range.
struct WaveLoop {
    const uint8_t* cbase;   // code plane of the tile
    const uint8_t* sbase;   // scale plane of the tile
    const _Float16* xrow;   // activations of this lane's token at its k-set (int8 formats)
    const uint8_t* xg;      // activations, M x K fp16 row-major (Q4_0)
    uint8_t* xs;            // this wave's staging area in LDS (Q4_0)
    uint32_t x_row;         // byte offset of this lane's token row in it (Q4_0)
    int M, K;
    uint32_t c_lane, c_unit, c_part, s_unit;
    uint32_t s_row[4];      // scale offsets of rows 4r .. 4r+3 (clamped)
    int ua, ub;             // units [ua, ub)
};

// Q4_0 activations go through LDS.  Read straight from memory, the A
// fragments of one unit take two load instructions that each touch 16 token
// rows (16 cache lines for 512 bytes).  Instead each wave copies the M token
// rows of its batch's K range (UNR units) into its own LDS area with
// global_load_lds (1 KB per instruction, a few lines each), then reads the
// fragments from there.  Row pitch: UNR * 4 + 1 chunks of 16 bytes (odd, so
// the 16 token rows of a fragment read fall in distinct banks).  Measured on
// the 151936 x 896 LM head: M = 8 / 16 from 23.2 / 29.5 to 20.5 / 22.5 us,
// M = 5 unchanged.  The int8 formats read one 16-byte fragment per unit, and
// staging them was 0.3-1 us slower on every shape measured.
template <int FMT, int UNR>
struct XStage {
    static constexpr int E = unit_elems(FMT);
    static constexpr int CPU = E / 8;                    // 16-byte chunks per unit and token
    static constexpr int P16 = UNR * CPU + 1;            // row pitch in chunks
    static constexpr int kChunks = (16 * P16 + 63) / 64 * 64;
    static constexpr int kBytes = kChunks * 16;          // per wave
};
template <int FMT>
constexpr bool staged_x() { return FMT == kQ4_0; }

// acc[m][i] += sum over the wave's units of w[4r+m, k] X[4j+i, k].  FULL: the
// tile has 64 rows, so the four scales of rows 4r..4r+3 are one load.  The
// choice is made once per workgroup so the load phase has no branches.
template <int FMT, int UNR, bool FULL>
__device__ __forceinline__ void accumulate(const WaveLoop& L, f32x4 (&acc)[4]) {
    constexpr int P = unit_parts(FMT);
    constexpr int SB = scale_bytes(FMT);
    constexpr int E = unit_elems(FMT);
    constexpr int KS = steps_of<FMT>();
    using XS = XStage<FMT, UNR>;
    for (int u = L.ua; u < L.ub; u += UNR) {
        if constexpr (staged_x<FMT>()) {
            // The batch's activations: lane l of copy i fills chunk
            // q = 64 i + l of the area: token row t = q / P16 (token
            // min(t, M - 1)), chunk kc of that row: unit min(u + kc / CPU,
            // ub - 1), its chunk kc % CPU.  The pad chunk and rows past M
            // re-read data nobody uses.
            const int ni = (L.M * XS::P16 + 63) / 64;
            for (int i = 0; i < ni; ++i) {
                const int q = 64 * i + (int(threadIdx.x) & 63);
                const int t = min(q / XS::P16, L.M - 1);
                const int kc = min(q % XS::P16, UNR * XS::CPU - 1);
                const int uk = min(u + kc / XS::CPU, L.ub - 1);
                const size_t off = size_t(t) * size_t(L.K) + size_t(uk) * E + size_t(kc % XS::CPU) * 8;
                __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(L.xg + 2 * off),
                                                 (__attribute__((address_space(3))) void*)(L.xs + 1024 * i), 16,
                                                 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        MUnit<FMT> b[UNR];
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
            if constexpr (!staged_x<FMT>()) {
                const _Float16* xp = L.xrow + size_t(uu) * E;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const u32x4 v = *reinterpret_cast<const u32x4*>(xp + 32 * ks);
                    b[k].xl[ks] = u32x2{v.x, v.y};
                    b[k].xh[ks] = u32x2{v.z, v.w};
                }
            }
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
        // Every load of the batch is issued before any of its data is used.
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (staged_x<FMT>()) {
            // The copies into LDS have landed once at most the batch's code
            // and scale loads (issued after them) are outstanding; then lane
            // (r, g) reads elements 4g .. 4g+3 and 16+4g .. of each unit from
            // its token's row.
            constexpr int kBatchLoads = UNR * (P + (FULL ? 1 : 4));
            static_assert(kBatchLoads <= 63, "vmcnt range");
            __builtin_amdgcn_s_waitcnt((kBatchLoads & 15) | (0x7 << 4) | (0xF << 8) | ((kBatchLoads >> 4) << 14));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < UNR; ++k) {
                const uint8_t* xp = L.xs + L.x_row + k * 64 + 8 * (int(threadIdx.x) >> 4 & 3);
                b[k].xl[0] = *reinterpret_cast<const u32x2*>(xp);
                b[k].xh[0] = *reinterpret_cast<const u32x2*>(xp + 32);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int k = 0; k < UNR; ++k) {
            if (u + k >= L.ub) continue;
            // Q4_0: t[0] slot m = code dword j of row 4r + m.  int8: t[2 ks]
            // and t[2 ks + 1] slot m = codes 8j .. 8j+3 and 8j+4 .. 8j+7 of
            // step ks of row 4r + m (a transpose of double dwords).
            u32x4 t[P];
            if constexpr (FMT == kQ4_0) {
                t[0] = xpose(b[k].c[0]);
            } else {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const u32x4 p0 = b[k].c[2 * ks], p1 = b[k].c[2 * ks + 1];
                    t[2 * ks] = xpose(u32x4{p0.x, p0.z, p1.x, p1.z});
                    t[2 * ks + 1] = xpose(u32x4{p0.y, p0.w, p1.y, p1.w});
                }
            }
            half8_t xa[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) xa[ks] = x_frag<FMT>(b[k].xl[ks], b[k].xh[ks]);
            // All four row groups' block sums first, then their scaling: an
            // FMA right behind the MFMA it reads would wait for its result.
            f32x4 sum[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                sum[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    half8_t wb;
                    if constexpr (FMT == kQ4_0) wb = q4_frag(t[0][m]);
                    else wb = i8_frag(t[2 * ks][m], t[2 * ks + 1][m]);
                    sum[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[ks], wb, sum[m], 0, 0, 0);
                }
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float d = scale_of<FMT, FULL>(b[k], m);
                acc[m] = __builtin_elementwise_fma(f32x4{d, d, d, d}, sum[m], acc[m]);
            }
        }
    }
}

// UNR: units whose loads one wave issues before computing them.
template <int FMT, int UNR>
__global__ __launch_bounds__(kGemvThreads) void gemv_multi_kernel(const MultiArgs a) {
    constexpr int UB = unit_bytes(FMT);
    constexpr int SB = scale_bytes(FMT);
    // One LDS area: the four waves' activation staging during the loop
    // (Q4_0), the cross-wave sums after it.
    constexpr int kStageBytes = staged_x<FMT>() ? 4 * XStage<FMT, UNR>::kBytes : 0;
    constexpr int kRedBytes = 4 * 16 * 64 * 4;
    __shared__ __attribute__((aligned(16))) uint8_t smem[kStageBytes > kRedBytes ? kStageBytes : kRedBytes];
    __shared__ uint32_t last;
    auto red = reinterpret_cast<float (*)[16][64]>(smem);

    const int bid = int(blockIdx.x);
    const MultiDesc& D = a.d[find_matrix(a.wg0, bid)];
    const int N = D.N, nu = D.nu, S = D.S, M = D.M, K = D.K;
    const int local = bid - D.wg0;
    // Every descriptor field the first loads need, in one scalar round trip
    // (the empty asm keeps the compiler from fetching the pointers after the
    // integers have returned).
    const uint8_t* const dcodes = D.codes;
    const uint8_t* const dscales = D.scales;
    const _Float16* const dx = D.x;
    const int tiles = D.tiles;
    asm volatile("" : : "s"(dcodes), "s"(dscales), "s"(dx), "s"(N), "s"(nu), "s"(S), "s"(M), "s"(K), "s"(tiles),
                 "s"(local));
    const int tile = int(uint32_t(local) / uint32_t(S));
    const int slice = local - tile * S;
    const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    const int lane = int(threadIdx.x) & 63;
    const int r = lane & 15, g = lane >> 4;
    const int nr = min(kTileRows, N - tile * kTileRows);
    const bool full = nr == kTileRows;

    int sa, sb;
    slice_units(nu, S, slice, sa, sb);
    const int ua = __builtin_amdgcn_readfirstlane(sa + int(uint32_t(sb - sa) * uint32_t(w) / 4));
    const int ub = __builtin_amdgcn_readfirstlane(sa + int(uint32_t(sb - sa) * uint32_t(w + 1) / 4));

    const size_t first = size_t(tile) * kTileRows * size_t(nu);
    WaveLoop L;
    L.cbase = dcodes + first * UB;
    L.sbase = dscales + first * SB;
    // Rows past the end of a partial tile are re-read from the last row and
    // never stored; so are tokens past M.
    L.c_lane = uint32_t(min(4 * r + g, nr - 1)) * 16u;
    L.c_unit = uint32_t(nr) * UB;
    L.c_part = uint32_t(nr) * 16u;
    L.s_unit = uint32_t(nr) * SB;
#pragma unroll
    for (int m = 0; m < 4; ++m) L.s_row[m] = uint32_t(min(4 * r + m, nr - 1)) * SB;
    // Q4_0 lane group g takes elements 4g..4g+3 and 16+4g.. of a block (the
    // nibbles of code dword g); int8 lane group g takes elements 8g..8g+7.
    L.xrow = dx + size_t(min(r, M - 1)) * size_t(K) + 8 * g;
    L.xg = reinterpret_cast<const uint8_t*>(dx);
    L.xs = smem + w * XStage<FMT, UNR>::kBytes;
    L.x_row = uint32_t(min(r, M - 1)) * uint32_t(XStage<FMT, UNR>::P16) * 16u;
    L.M = M;
    L.K = K;
    L.ua = ua;
    L.ub = ub;

    f32x4 acc[4] = {};
    if (full) accumulate<FMT, UNR, true>(L, acc);
    else accumulate<FMT, UNR, false>(L, acc);

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
            float* yp = D.y + size_t(token) * size_t(N) + row0;
            if (D.vec_y && full) {
                *reinterpret_cast<f32x4*>(yp) = f32x4{v[0], v[1], v[2], v[3]};
            } else {
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    if (4 * r + m < nr) yp[m] = v[m];
            }
        }
        return;
    }
    // Split K: publish this slice, then the last workgroup to arrive adds the
    // slices in slice order (lq_splitk.h).
    const size_t pitch = size_t(tiles) * kTileRows;   // floats per token of one slice
    const size_t spitch = pitch * size_t(M);             // floats per slice
    if (token < M) {
        float* pp = D.part + size_t(slice) * spitch + size_t(token) * pitch + row0;
#pragma unroll
        for (int m = 0; m < 4; ++m) splitk_put(pp + m, v[m]);
    }
    splitk_publish();
    __syncthreads();
    if (threadIdx.x == 0) last = splitk_arrive(&D.cnt[tile], a.tag, S) ? 1u : 0u;
    __syncthreads();
    if (!last) return;
    if (token < M) {
        const float* pp = D.part + size_t(token) * pitch + row0;
        float* yp = D.y + size_t(token) * size_t(N) + row0;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float t = sum_slices(pp + m, spitch, S);
            if (4 * r + m < nr) yp[m] = t;
        }
    }
}

}  // namespace

// Fewest and most units that the waves of a launch loop over: per matrix,
// ceil(ceil(nu / S) / 4) (the waves of one slice differ by at most one).
static void wave_units(const MultiArgs& a, int& least, int& most) {
    least = INT32_MAX;
    most = 0;
    for (int i = 0; i < a.count; ++i) {
        const int slice = (a.d[i].nu + a.d[i].S - 1) / a.d[i].S;
        least = min(least, (slice + 3) / 4);
        most = max(most, (slice + 3) / 4);
    }
}

hipError_t launch_gemv_multi(int fmt, const MultiArgs& a, hipStream_t stream) {
    const dim3 grid(unsigned(a.total_wgs)), block(kGemvThreads);
    switch (fmt) {
        case kQ4_0: {
            int least, most;
            wave_units(a, least, most);
            if (least > LQ_MULTI_UNR_Q4 && most <= LQ_MULTI_UNR_Q4_ONE)
                hipLaunchKernelGGL((gemv_multi_kernel<kQ4_0, LQ_MULTI_UNR_Q4_ONE>), grid, block, 0, stream, a);
            else
                hipLaunchKernelGGL((gemv_multi_kernel<kQ4_0, LQ_MULTI_UNR_Q4>), grid, block, 0, stream, a);
            break;
        }
        case kQ8_0: hipLaunchKernelGGL((gemv_multi_kernel<kQ8_0, LQ_MULTI_UNR_Q8>), grid, block, 0, stream, a); break;
        case kI8B64: hipLaunchKernelGGL((gemv_multi_kernel<kI8B64, LQ_MULTI_UNR_I8>), grid, block, 0, stream, a); break;
        case kI8B32: hipLaunchKernelGGL((gemv_multi_kernel<kI8B32, LQ_MULTI_UNR_Q8>), grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace lq
