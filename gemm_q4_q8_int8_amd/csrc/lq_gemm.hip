// Prefill GEMM for Q4_0 weights: Y[M x N] = X[M x K] * W[N x K]^T.
//
// Prefill is compute-bound ("oxinfer" page, "Performance"), and the GPU
// kernels the page describes dequantize the weight tile on chip before the
// dense contraction ("Platforms and accelerators": weights dequantized in
// threadgroup memory).  On gfx950 the dense step is the fp16 matrix-core
// instruction v_mfma_f32_32x32x16_f16 (fp32 accumulate), so weights are
// rounded once to fp16: RN_fp16((q - 8) * d).
//
// Design for gfx950 (measured here: ds_read_b128 ~220 B/clk/CU, fp16 MFMA
// ~36 cycles per 32x32x16 instruction, and a wave's vector ALU work does not
// overlap its own matrix instructions, so two waves per SIMD are needed):
//   * A workgroup of 8 waves owns a 256 x 128 output tile; wave (wm, wn)
//     owns rows 64 wm .. +64 and columns 64 wn .. +64 (2 x 2 blocks of
//     32 x 32 fp32 accumulators).  One step is one Q4_0 block (32 of K).
//   * A copy ring of six LDS slots is filled with global_load_lds (straight
//     to LDS, no registers), four steps ahead: the step's X tile (256 rows x
//     32 fp16, 16-byte chunks XOR-swizzled by row so fragment reads and
//     copies are free of bank conflicts) and the raw codes and scales of
//     the block for the workgroup's two 64-row packed tiles (contiguous 1 KB
//     runs in the packed layout).
//   * While the matrix instructions of step st run, the 512 threads unpack
//     step st + 2's weights once per workgroup into an fp16 B tile (triple
//     buffered) and read the A and B fragments of step st + 1: v_perm_b32
//     places each nibble under the fp16 exponent 2^10, v_pk_add_f16 removes
//     1032 (exact q - 8) and v_pk_mul_f16 applies d with one rounding.  One
//     barrier per step.
//   * Few output tiles (the 2048 x 11008 down projection has 32) split K
//     across workgroups: each slice writes its partial tile to the caller's
//     workspace and a second kernel adds the slices in order (deterministic).
//   * Workgroups that read the same weights (same N tile, different M tile)
//     are placed on the same XCD so the second read hits that XCD's L2.
//   * The epilogue stages the tile through LDS so stores are whole rows.
#include "lq_internal.h"

#include <algorithm>
#include <atomic>

namespace lq {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256;
constexpr int BN = 128;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
// One ring slot: X (256 rows x 64 B), the codes of one block of the two
// packed tiles (2 x 1 KB), their scales (2 x 256 B: a 2-byte load to LDS
// fills one dword per lane, zero-extended), and 256 B that absorb the extra
// loads of waves with nothing else to copy.
constexpr int kXRowBytes = 64;
constexpr int kWOff = BM * kXRowBytes;            // 16,384
constexpr int kSOff = kWOff + 2 * 1024;           // 18,432
constexpr int kDummyOff = kSOff + 2 * 256;        // 18,944
constexpr int kSlotBytes = kDummyOff + 256;       // 19,200
constexpr int kStages = 6;                        // loads run four steps ahead
constexpr int kLoadsPerStep = 3;                  // per wave: 2 X + 1 code/scale/dummy
constexpr int kBTileBytes = BN * 64;              // fp16 B tile: 128 columns x 32
constexpr int kBOff = kStages * kSlotBytes;       // 115,200
constexpr int kLdsBytes = kBOff + 3 * kBTileBytes;   // 139,776 B of the 160 KB
// Output tiles below which K is split across workgroups, and the workgroups
// a split aims for.
constexpr int kSplitBelowTiles = 128;
constexpr int kSplitTargetWgs = 256;

struct GemmArgs {
    const uint8_t* codes;     // code plane (tiled layout)
    const uint16_t* scales;   // scale plane (tiled layout)
    const _Float16* X;        // M x K row-major
    float* out;               // Y (S == 1) or S partial M x N slices
    int32_t M, N, K, nu;      // nu = K / 32
    int32_t tiles_m, tiles_n, S, us;   // us: blocks per K slice
    int32_t remap;            // 1: XCD-aware workgroup order
    int32_t pad;
};

__device__ __forceinline__ uint32_t bits(half2_t h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ half2_t as_half2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// Two fp16 weights RN_fp16((q - 8) * d) from two nibbles (bytes `sel` of v).
__device__ __forceinline__ uint32_t w2(uint32_t v, uint32_t sel, half2_t dd) {
    const half2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
    return bits((as_half2(__builtin_amdgcn_perm(0x64646464u, v, sel)) - off) * dd);
}

// LDS byte offset of 16-byte chunk `chunk` (0-3) of a 64-byte row (an X row
// or a B column).  XORing the chunk with bits 2-3 of the row makes the 16
// lanes of one LDS cycle (64 banks) hit 16 distinct (row % 4, chunk) slots
// both for fragment reads (16 rows, one chunk) and for row writes.
__device__ __forceinline__ uint32_t sw_off(int row, int chunk) {
    return uint32_t(row) * 64u + uint32_t((chunk ^ ((row >> 2) & 3)) * 16);
}

// Workgroup barrier that orders LDS accesses (a compiler memory barrier) but
// adds no wait of its own: __syncthreads() would also wait for every
// outstanding global load, including the copy-ring loads of later steps that
// are meant to stay in flight across it.  Callers wait for what they need.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS accesses done
    asm volatile("s_barrier" ::: "memory");
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// of this wave are outstanding (lgkm and exp counters left unconstrained).
constexpr int vmcnt_imm(int n) { return (n & 15) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14); }

__global__ __launch_bounds__(kThreads, 1) void gemm_q4_0_kernel(const GemmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    // Work item: M tile fastest, then N tile, then K slice.
    int L = blockIdx.x;
    if (a.remap) L = (L % 8) * int(gridDim.x / 8) + L / 8;
    const int tm = L % a.tiles_m;
    const int rest = L / a.tiles_m;
    const int tn = rest % a.tiles_n;
    const int ks = rest / a.tiles_n;
    const int m0 = tm * BM;
    const int u0 = ks * a.us;
    const int nst = min(a.nu, u0 + a.us) - u0;   // steps (blocks) of this slice

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5;
    const int tiles_b = (a.N + kTileRows - 1) / kTileRows;

    // ---- copy ring.  Per step each wave issues kLoadsPerStep loads:
    //   X: wave w covers rows 32 w .. +32 in two 1 KB loads; lane s of load
    //      i fills row 32 w + 16 i + s / 4, physical chunk s % 4, i.e.
    //      logical chunk (s % 4) ^ ((row >> 2) & 3).
    //   waves 0-1: the block's codes of packed tile 2 tn + w (lane s: row s,
    //      clamped into the tile); waves 2-3: its scales; waves 4-7: a spare
    //      load of scales into the slot's dummy area (keeps the per-wave
    //      count uniform for the wait).
    uint32_t xo[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = 32 * wave + 16 * i + (lane >> 2);
        const int c = (lane & 3) ^ ((row >> 2) & 3);
        xo[i] = uint32_t(min(m0 + row, a.M - 1)) * uint32_t(a.K) * 2u + uint32_t(c) * 16u;
    }
    const int lt = wave & 1;
    const int ltb = min(tn * 2 + lt, tiles_b - 1);
    const int lnr = min(kTileRows, a.N - ltb * kTileRows);
    const uint8_t* lcode = a.codes + size_t(ltb) * kTileRows * size_t(a.nu) * 16;
    const uint16_t* lscale = a.scales + size_t(ltb) * kTileRows * size_t(a.nu);
    const uint32_t lrow = uint32_t(min(lane, lnr - 1));
    auto issue = [&](int st) {   // loads of step st into slot st % kStages
        uint8_t* slot = lds + (st % kStages) * kSlotBytes;
        const int ub = u0 + st;
        const uint8_t* xb = reinterpret_cast<const uint8_t*>(a.X) + size_t(ub) * 64;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(xb + xo[i]),
                (__attribute__((address_space(3))) void*)(slot + (2 * wave + i) * 1024), 16, 0, 0);
        const size_t e = size_t(ub) * size_t(lnr) + lrow;
        if (wave < 2)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(lcode + e * 16),
                (__attribute__((address_space(3))) void*)(slot + kWOff + lt * 1024), 16, 0, 0);
        else
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(lscale + e),
                (__attribute__((address_space(3))) void*)(slot + (wave < 4 ? kSOff + lt * 256 : kDummyOff)), 2, 0, 0);
    };

    // ---- unpack: thread t turns 8 weights of column n = t / 4 into one
    // 16-byte chunk of the fp16 B tile: part p = t % 4 takes elements
    // 8p .. 8p + 7 of the block, i.e. the low (p < 2) or high (p >= 2)
    // nibbles of code bytes 8 (p % 2) .. 8 (p % 2) + 7 (GGUF order).
    const int un = tid >> 2, up = tid & 3;
    const uint32_t uc_off = uint32_t(kWOff + (un >> 6) * 1024 + (un & 63) * 16 + 8 * (up & 1));
    const uint32_t us_off = uint32_t(kSOff + (un >> 6) * 256 + (un & 63) * 4);
    const uint32_t ub_off = sw_off(un, up);
    auto unpack = [&](const uint8_t* slot, uint8_t* btile) {
        const u32x2 c = *reinterpret_cast<const u32x2*>(slot + uc_off);
        const uint16_t d = *reinterpret_cast<const uint16_t*>(slot + us_off);
        const _Float16 dh = __builtin_bit_cast(_Float16, d);
        const half2_t dd = {dh, dh};
        const int sh = (up >> 1) * 4;
        const uint32_t n0 = (c.x >> sh) & 0x0F0F0F0Fu, n1 = (c.y >> sh) & 0x0F0F0F0Fu;
        const u32x4 v = {w2(n0, 0x04010400u, dd), w2(n0, 0x04030402u, dd), w2(n1, 0x04010400u, dd),
                         w2(n1, 0x04030402u, dd)};
        *reinterpret_cast<u32x4*>(btile + ub_off) = v;
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // ---- main loop, software-pipelined over three steps: at step st the
    // matrix instructions of step st run on fragments read during step
    // st - 1, the fragments of step st + 1 are read, and the weights of step
    // st + 2 are unpacked (B tiles are triple-buffered), so LDS latency and
    // unpacking overlap the matrix instructions instead of following a
    // barrier.  Copies run three steps ahead of the unpacking: at the top of
    // step st the loads of steps up to st + 2 have landed, st + 3 and st + 4
    // may be in flight, and st + 5 is issued (clamped to the last step: past
    // the end the copy lands in a slot nobody reads, so every step issues the
    // same number of loads and the wait count is a constant).
    auto slot_of = [&](int st) { return lds + (st % kStages) * kSlotBytes; };
    auto btile_of = [&](int st) { return lds + kBOff + (st % 3) * kBTileBytes; };
    half8_t af[2][2], bf[2][2];   // [sub-step][block] of the next step to multiply
    auto read_frags = [&](int st) {
        const uint8_t* slot = slot_of(st);
        const uint8_t* bt = btile_of(st);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                af[s][i] = *reinterpret_cast<const half8_t*>(slot + sw_off(wm * 64 + i * 32 + (lane & 31), 2 * s + h));
                bf[s][i] = *reinterpret_cast<const half8_t*>(bt + sw_off(wn * 64 + i * 32 + (lane & 31), 2 * s + h));
            }
    };
    if (nst > 0) {
#pragma unroll
        for (int p = 0; p < kStages - 1; ++p) issue(min(p, nst - 1));
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((kStages - 3) * kLoadsPerStep));   // steps 0, 1 landed
        lds_barrier();
        unpack(slot_of(0), btile_of(0));
        unpack(slot_of(1), btile_of(1));
        lds_barrier();
        read_frags(0);
    }
    for (int st = 0; st < nst; ++st) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kLoadsPerStep));   // step st + 2 landed
        lds_barrier();
        issue(min(st + kStages - 1, nst - 1));
        unpack(slot_of(st + 2), btile_of(st + 2));   // past the last step: unused data
        half8_t a0[2][2], b0[2][2];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                a0[s][i] = af[s][i];
                b0[s][i] = bf[s][i];
            }
        read_frags(st + 1);                          // past the last step: unused data
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[s][i], b0[s][j], acc[i][j], 0, 0, 0);
    }

    // ---- epilogue: the tile goes through LDS in two halves of 128 rows so
    // global stores are whole 512-byte rows, 16 bytes per lane.  32x32
    // accumulator layout: register r of lane l is row 8 (r / 4) + 4 (l / 32)
    // + r % 4, column l % 32.  Row pitch 136 floats: the two half waves
    // (rows 4 apart) write disjoint banks.
    constexpr int kCPitch = BN + 8;
    float* cst = reinterpret_cast<float*>(lds);
    float* out = a.out + size_t(ks) * size_t(a.M) * size_t(a.N);
    const int n0 = tn * BN;
    const int col = (tid & 31) * 4;
    const bool full = m0 + BM <= a.M && n0 + BN <= a.N && (a.N & 3) == 0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        __syncthreads();
        if ((wm >> 1) == half) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = (wm & 1) * 64 + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                        cst[row * kCPitch + wn * 64 + j * 32 + (lane & 31)] = acc[i][j][r];
                    }
        }
        __syncthreads();
#pragma unroll 4
        for (int k = 0; k < 8; ++k) {
            const int row = (tid >> 5) + 16 * k;
            const f32x4 v = *reinterpret_cast<const f32x4*>(cst + row * kCPitch + col);
            const int m = m0 + half * 128 + row;
            if (full) {
                *reinterpret_cast<f32x4*>(out + size_t(m) * size_t(a.N) + n0 + col) = v;
            } else if (m < a.M) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n0 + col + e < a.N) out[size_t(m) * size_t(a.N) + n0 + col + e] = v[e];
            }
        }
    }
}

// Y = sum of the S partial slices, added in slice order.
__global__ __launch_bounds__(256) void splitk_reduce(const float* __restrict__ P, float* __restrict__ Y,
                                                     size_t mn, int S) {
    const size_t i4 = (size_t(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (i4 >= mn) return;
    if (i4 + 4 <= mn) {
        f32x4 t = *reinterpret_cast<const f32x4*>(P + i4);
        for (int s = 1; s < S; ++s) t += *reinterpret_cast<const f32x4*>(P + size_t(s) * mn + i4);
        *reinterpret_cast<f32x4*>(Y + i4) = t;
    } else {
        for (size_t i = i4; i < mn; ++i) {
            float t = P[i];
            for (int s = 1; s < S; ++s) t += P[size_t(s) * mn + i];
            Y[i] = t;
        }
    }
}

struct Plan {
    int tiles_m, tiles_n, S, us;
};

Plan plan_gemm(int64_t M, int64_t N, int64_t K) {
    Plan p;
    p.tiles_m = int((M + BM - 1) / BM);
    p.tiles_n = int((N + BN - 1) / BN);
    const int nu = int(K / 32);
    const int64_t tiles = int64_t(p.tiles_m) * p.tiles_n;
    int S = 1;
    if (tiles < kSplitBelowTiles) S = int(std::max<int64_t>(1, kSplitTargetWgs / tiles));
    S = std::min(S, std::max(1, nu / 16));   // at least 16 blocks (steps) per slice
    const int us = (nu + S - 1) / S;
    p.us = us;
    p.S = (nu + us - 1) / us;                // no empty slice
    return p;
}

}  // namespace

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const Plan p = plan_gemm(M, N, K);
    return p.S > 1 ? size_t(p.S) * size_t(M) * size_t(N) * sizeof(float) : 0;
}

hipError_t launch_splitk_reduce(const float* P, float* Y, size_t mn, int S, hipStream_t stream) {
    const size_t blocks = (mn + 1023) / 1024;
    hipLaunchKernelGGL(splitk_reduce, dim3(unsigned(blocks)), dim3(256), 0, stream, P, Y, mn, S);
    return hipGetLastError();
}

hipError_t launch_gemm_q4_0(const void* W, const void* X, float* Y, int64_t M, int64_t N,
                            int64_t K, void* ws, size_t, int, hipStream_t stream) {
    const Plan p = plan_gemm(M, N, K);
    GemmArgs a;
    a.codes = static_cast<const uint8_t*>(W);
    a.scales = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(W) +
                                                 align256(code_plane_bytes(kQ4_0, N, K)));
    a.X = static_cast<const _Float16*>(X);
    a.out = p.S > 1 ? static_cast<float*>(ws) : Y;
    a.M = int32_t(M);
    a.N = int32_t(N);
    a.K = int32_t(K);
    a.nu = int32_t(K / 32);
    a.tiles_m = p.tiles_m;
    a.tiles_n = p.tiles_n;
    a.S = p.S;
    a.us = p.us;
    const int64_t grid = int64_t(p.tiles_m) * p.tiles_n * p.S;
    a.remap = (grid % 8 == 0) ? 1 : 0;
    a.pad = 0;
    // The ring needs more than the default 64 KB of dynamic LDS: raise the
    // kernel's limit once per device.
    int dev = 0;
    hipError_t e0 = hipGetDevice(&dev);
    if (e0 != hipSuccess) return e0;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    static std::atomic<bool> lds_ok[64];
    if (!lds_ok[dev].load(std::memory_order_acquire)) {
        e0 = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_q4_0_kernel),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
        if (e0 != hipSuccess) return e0;
        lds_ok[dev].store(true, std::memory_order_release);
    }
    hipLaunchKernelGGL(gemm_q4_0_kernel, dim3(unsigned(grid)), dim3(kThreads), kLdsBytes, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.S == 1) return e;
    return launch_splitk_reduce(static_cast<const float*>(ws), Y, size_t(M) * size_t(N), p.S, stream);
}

}  // namespace lq
