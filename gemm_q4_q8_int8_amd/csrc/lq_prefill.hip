// Prefill GEMM for int8-coded weights (Q8_0 and int8 block-64):
// Y[M x N] = X[M x K] W[N x K]^T, fp16 X, weights read straight from the
// packed layout into matrix-core operands.
//
// Prefill is compute bound ("oxinfer" page, "Performance"); the page's GPU
// kernels dequantize the weight tile on chip before a dense tile product
// ("Platforms and accelerators").  Here the dense step is
// v_mfma_f32_16x16x32_f16 and the weight tile never passes through LDS in
// unpacked form:
//   * A workgroup of 4 waves owns 256 weight rows (4 packed 64-row tiles, one
//     per wave) x 64 tokens (NT = 4 groups of 16); one step is 32 elements of
//     K.  (128 tokens per workgroup was measured too: fewer workgroups for
//     the same output, no faster.)
//   * A ring of LDS slots is filled with global_load_lds several steps
//     ahead.  A slot holds the step's 64 x 32 fp16 activation block (rows of
//     64 bytes, 16-byte chunks XOR-swizzled by token so that fragment reads
//     are free of bank conflicts), the raw code bytes of the 4 tiles and
//     their scales.  Each wave copies its own tile's codes and a quarter of
//     the activations; one barrier per step.
//   * Each wave reads its tile's codes for the step (two 16-byte LDS reads,
//     lane (r, g) holding tile row 4r + g), transposes them across the four
//     16-lane rows with permlane swaps (as double dwords) so that lane (r, j)
//     holds codes 8j .. 8j+7 of rows 4r .. 4r+3, and turns them into fp16 B
//     fragments in registers.  Its activation fragment is one 16-byte read
//     of elements 8j .. 8j+7; the four waves share the slot's activations.
//   * Q8_0: the B fragment is RN_fp16(c d) (exact fp16 code, one fp16
//     multiply by the fp16 scale), the fp16 tile contract of lq_dequant_f16,
//     and the 16 matrix instructions of a step accumulate straight into the
//     fp32 tile.  int8 block-64: the fp32 scale is not an fp16 value, so the
//     codes stay exact and the scale is applied in fp32 to each step's
//     block sums (more accurate than an fp16 tile).
//   * Short K slices per output tile split K across workgroups into the
//     caller's workspace; a second kernel adds the slices in order.
//   * Q4_0 weights use the LDS-tile GEMM: this design was measured on them
//     too (nibbles selected per lane group) and was slower on the 11008-row
//     matrices (474 against 547 TFLOP/s).
#include "lq_frag.h"

#include <algorithm>
#include <atomic>

namespace lq {
namespace {

using namespace frag;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// 16-token groups per workgroup (tokens per workgroup = 16 NT).
#ifndef LQ_PREFILL_NT
#define LQ_PREFILL_NT 4
#endif
constexpr int NT = LQ_PREFILL_NT;
constexpr int kTok = 16 * NT;

// Slot geometry per format: X block (16 NT tokens x 64 bytes), code parts of the
// step for the four tiles (1 KB each), scales (one dword per row: a 2-byte
// copy to LDS fills a zero-extended dword).
template <int FMT>
struct Cfg {
    static constexpr int PS = 2;                       // 16-byte code parts per step
    static constexpr int XOFF = 0;
    static constexpr int WOFF = kTok * 64;             // 64 bytes per token
    static constexpr int SOFF = WOFF + kWaves * PS * 1024;
    static constexpr int SLOT = SOFF + kWaves * 256;
    static constexpr int STAGES = NT == 4 ? 6 : 4;
    static constexpr int LDS = STAGES * SLOT;         // at most 80 KB: two workgroups per CU
    static constexpr int XL = NT / 4;                 // activation copies per wave per step
    static constexpr int LOADS = XL + PS + 1;          // copies per wave per step
};

struct PrefillArgs {
    const uint8_t* codes;    // code plane (tiled)
    const uint8_t* scales;   // scale plane (tiled)
    const _Float16* X;       // M x K row-major
    float* out;              // Y (S == 1) or S partial M x N slices
    int32_t M, N, K, nu;     // nu: units per row
    int32_t tiles;           // 64-row packed tiles
    int32_t rb, tb, S, us;   // row blocks, token blocks, K slices, steps per slice
    int32_t remap;           // 1: XCD-aware workgroup order
    int32_t vec;             // Y rows 16-byte aligned (N % 4 == 0)
};

__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS accesses done
    asm volatile("s_barrier" ::: "memory");
}

constexpr int vmcnt_imm(int n) { return (n & 15) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14); }

template <int FMT>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(const PrefillArgs a) {
    using C = Cfg<FMT>;
    constexpr int SB = scale_bytes(FMT);
    constexpr int UB = unit_bytes(FMT);
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    // Work item: token block fastest, then row block, then K slice; with the
    // remap, consecutive items share an XCD (and its L2) and so mostly the
    // same weight rows.
    int L = blockIdx.x;
    if (a.remap) L = (L % 8) * int(gridDim.x / 8) + L / 8;
    const int tb = L % a.tb;
    const int rest = L / a.tb;
    const int rb = rest % a.rb;
    const int ks = rest / a.rb;
    const int nsteps = a.K / 32;
    const int s0 = ks * a.us;
    const int nst = min(nsteps, s0 + a.us) - s0;
    const int t0 = tb * kTok;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;

    // This wave's packed tile (clamped: a row block past the last tile
    // recomputes the last one and stores nothing).
    const int tile = min(rb * kWaves + w, a.tiles - 1);
    const int nr = min(kTileRows, a.N - tile * kTileRows);
    const size_t first = size_t(tile) * kTileRows * size_t(a.nu);
    const uint8_t* tcodes = a.codes + first * UB;
    const uint8_t* tscales = a.scales + first * SB;
    const uint32_t w_lane = uint32_t(min(4 * r + g, nr - 1)) * 16u;   // code copy: tile row 4r + g
    const uint32_t s_lane = uint32_t(min(lane, nr - 1)) * SB;          // scale copy: tile row `lane`

    // Activation copies: copy i of lane s of wave w fills token
    // 16 (XL w + i) + s / 4, physical chunk s % 4 of that token's 64-byte
    // row, i.e. logical chunk (s % 4) ^ ((token >> 2) & 3).
    const uint8_t* xsrc[C::XL];
#pragma unroll
    for (int i = 0; i < C::XL; ++i) {
        const int xtok = 16 * (C::XL * w + i) + (lane >> 2);
        const int xlc = (lane & 3) ^ ((xtok >> 2) & 3);
        xsrc[i] = reinterpret_cast<const uint8_t*>(a.X) +
                  (size_t(min(t0 + xtok, a.M - 1)) * size_t(a.K) + size_t(8 * xlc)) * 2;
    }

    auto slot_of = [&](int st) { return lds + (st % C::STAGES) * C::SLOT; };
    auto issue = [&](int st) {
        uint8_t* slot = slot_of(st);
        const int step = s0 + st;
#pragma unroll
        for (int i = 0; i < C::XL; ++i)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(xsrc[i] + size_t(step) * 64),
                (__attribute__((address_space(3))) void*)(slot + C::XOFF + (C::XL * w + i) * 1024), 16, 0, 0);
        const int u = FMT == kI8B64 ? step >> 1 : step;
        const int p0 = FMT == kI8B64 ? 2 * (step & 1) : 0;
        const uint8_t* cu = tcodes + size_t(u) * nr * UB + w_lane;
#pragma unroll
        for (int p = 0; p < C::PS; ++p)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(cu + size_t(p0 + p) * nr * 16),
                (__attribute__((address_space(3))) void*)(slot + C::WOFF + (w * C::PS + p) * 1024), 16, 0, 0);
        const auto* ssrc = (const __attribute__((address_space(1))) void*)(tscales + size_t(u) * nr * SB + s_lane);
        auto* sdst = (__attribute__((address_space(3))) void*)(slot + C::SOFF + w * 256);
        if constexpr (SB == 2) __builtin_amdgcn_global_load_lds(ssrc, sdst, 2, 0, 0);
        else __builtin_amdgcn_global_load_lds(ssrc, sdst, 4, 0, 0);
    };

    // Fragment offsets inside a slot: token group q, lane (t, j) takes
    // elements 8j .. 8j+7 of token 16 q + t, i.e. logical chunk j, one 16-byte
    // read (16 tokens x one chunk: conflict-free under the swizzle).
    uint32_t xoff[NT];
#pragma unroll
    for (int q = 0; q < NT; ++q) {
        const int tok = 16 * q + r;
        const int sw = (tok >> 2) & 3;
        xoff[q] = uint32_t(C::XOFF + tok * 64 + (g ^ sw) * 16);
    }
    const uint32_t woff = uint32_t(C::WOFF + w * C::PS * 1024 + 16 * lane);
    const uint32_t soff = uint32_t(C::SOFF + w * 256 + 16 * r);

    f32x4 acc[NT][4];
#pragma unroll
    for (int q = 0; q < NT; ++q)
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[q][m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    if (nst > 0) {
#pragma unroll
        for (int p = 0; p < C::STAGES - 1; ++p) issue(min(p, nst - 1));
    }
    for (int st = 0; st < nst; ++st) {
        // Step st's copies (this wave's) have landed once at most the later
        // STAGES - 2 steps' copies are outstanding; the barrier makes every
        // wave's copies visible and frees the slot of step st - 1.
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((C::STAGES - 2) * C::LOADS));
        lds_barrier();
        issue(min(st + C::STAGES - 1, nst - 1));
        const uint8_t* slot = slot_of(st);
        // Lane (r, j), slot m: the codes of elements 8j .. 8j+7 of row 4r + m
        // in c[0] (first four) and c[1] (last four), by a transpose of double
        // dwords.
        u32x4 c[2];
        half8_t xa[NT];
        const u32x4 p0 = *reinterpret_cast<const u32x4*>(slot + woff);
        const u32x4 p1 = *reinterpret_cast<const u32x4*>(slot + woff + 1024);
        c[0] = xpose(u32x4{p0.x, p0.z, p1.x, p1.z});
        c[1] = xpose(u32x4{p0.y, p0.w, p1.y, p1.w});
#pragma unroll
        for (int q = 0; q < NT; ++q) xa[q] = *reinterpret_cast<const half8_t*>(slot + xoff[q]);
        const u32x4 sc = *reinterpret_cast<const u32x4*>(slot + soff);
        const uint32_t sv[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            if constexpr (FMT == kI8B64) {
                const half8_t wb = i8_frag(c[0][m], c[1][m]);
                const float s = __uint_as_float(sv[m]);
#pragma unroll
                for (int q = 0; q < NT; ++q) {
                    const f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[q], wb, f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                    acc[q][m] = __builtin_elementwise_fma(f32x4{s, s, s, s}, t, acc[q][m]);
                }
            } else {
                const _Float16 d = __builtin_bit_cast(_Float16, uint16_t(sv[m]));
                const half8_t dd = {d, d, d, d, d, d, d, d};
                const half8_t wb = i8_frag(c[0][m], c[1][m]) * dd;
#pragma unroll
                for (int q = 0; q < NT; ++q)
                    acc[q][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[q], wb, acc[q][m], 0, 0, 0);
            }
        }
    }

    // Lane (r, j) holds, for token group q, tokens 16q + 4j + i of weight rows
    // 4r .. 4r+3 of this wave's tile: four consecutive columns of Y.
    if (rb * kWaves + w >= a.tiles) return;
    float* out = a.out + size_t(ks) * size_t(a.M) * size_t(a.N);
    const int n0 = tile * kTileRows + 4 * r;
    const bool vec = a.vec && 4 * r + 4 <= nr;
#pragma unroll
    for (int q = 0; q < NT; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = t0 + 16 * q + 4 * g + i;
            if (tok >= a.M) continue;
            float* yp = out + size_t(tok) * size_t(a.N) + n0;
            if (vec) {
                *reinterpret_cast<f32x4*>(yp) = f32x4{acc[q][0][i], acc[q][1][i], acc[q][2][i], acc[q][3][i]};
            } else {
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    if (4 * r + m < nr) yp[m] = acc[q][m][i];
            }
        }
}

struct Plan {
    int rb, tb, S, us;
};

// Split K when the output has fewer work items than about two workgroups
// per CU of a 256-CU part, keeping at least 16 steps (512 elements of K) per
// slice.  A fixed target keeps the plan (and the workspace size) independent
// of the device.
#ifndef LQ_PREFILL_TARGET_WGS
#define LQ_PREFILL_TARGET_WGS 512
#endif
constexpr int64_t kTargetWgs = LQ_PREFILL_TARGET_WGS;
#ifndef LQ_PREFILL_SPLIT_BELOW
#define LQ_PREFILL_SPLIT_BELOW 256
#endif
constexpr int64_t kSplitBelow = LQ_PREFILL_SPLIT_BELOW;
Plan plan(int64_t M, int64_t N, int64_t K) {
    Plan p;
    const int64_t tiles = (N + kTileRows - 1) / kTileRows;
    p.rb = int((tiles + kWaves - 1) / kWaves);
    p.tb = int((M + kTok - 1) / kTok);
    const int nsteps = int(K / 32);
    const int64_t items = int64_t(p.rb) * p.tb;
    // Partial slices cost their M x N floats twice more in memory traffic, so
    // K is split only when the output alone leaves most CUs idle.
    int S = 1;
    if (items < kSplitBelow) S = int((kTargetWgs + items - 1) / items);
    S = std::min(S, std::max(1, nsteps / 16));
    p.us = (nsteps + S - 1) / S;
    p.S = (nsteps + p.us - 1) / p.us;
    return p;
}

template <int FMT>
hipError_t launch_fmt(const PrefillArgs& a, int64_t grid, hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    static std::atomic<bool> lds_ok[64];
    if (!lds_ok[dev].load(std::memory_order_acquire)) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<FMT>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, Cfg<FMT>::LDS);
        if (e != hipSuccess) return e;
        lds_ok[dev].store(true, std::memory_order_release);
    }
    hipLaunchKernelGGL(prefill_kernel<FMT>, dim3(unsigned(grid)), dim3(kThreads), Cfg<FMT>::LDS, stream, a);
    return hipGetLastError();
}

}  // namespace

size_t prefill_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const Plan p = plan(M, N, K);
    return p.S > 1 ? size_t(p.S) * size_t(M) * size_t(N) * sizeof(float) : 0;
}

hipError_t launch_prefill(int fmt, const void* W, const void* X, float* Y, int64_t M, int64_t N,
                          int64_t K, void* ws, hipStream_t stream) {
    const Plan p = plan(M, N, K);
    PrefillArgs a;
    a.codes = static_cast<const uint8_t*>(W);
    a.scales = static_cast<const uint8_t*>(W) + align256(code_plane_bytes(fmt, N, K));
    a.X = static_cast<const _Float16*>(X);
    a.out = p.S > 1 ? static_cast<float*>(ws) : Y;
    a.M = int32_t(M);
    a.N = int32_t(N);
    a.K = int32_t(K);
    a.nu = int32_t(K / unit_elems(fmt));
    a.tiles = int32_t((N + kTileRows - 1) / kTileRows);
    a.rb = p.rb;
    a.tb = p.tb;
    a.S = p.S;
    a.us = p.us;
    const int64_t grid = int64_t(p.rb) * p.tb * p.S;
    a.remap = (grid % 8 == 0) ? 1 : 0;
    a.vec = (N % 4 == 0 && reinterpret_cast<uintptr_t>(a.out) % 16 == 0) ? 1 : 0;
    hipError_t e;
    switch (fmt) {
        case kQ8_0: e = launch_fmt<kQ8_0>(a, grid, stream); break;
        case kI8B64: e = launch_fmt<kI8B64>(a, grid, stream); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || p.S == 1) return e;
    return launch_splitk_reduce(static_cast<const float*>(ws), Y, size_t(M) * size_t(N), p.S, stream);
}

}  // namespace lq
