// Prefill GEMM for Q4_0 weights: Y[M x N] = X[M x K] * W[N x K]^T.
//
// Prefill is compute-bound ("oxinfer" page, "Performance"), and the GPU
// kernels the page describes dequantize the weight tile on chip before the
// dense contraction ("Platforms and accelerators": weights dequantized in
// threadgroup memory).  On gfx950 the dense step is the fp16 matrix-core
// instruction v_mfma_f32_32x32x16_f16 (fp32 accumulate), so weights are
// rounded once to fp16: RN_fp16((q - 8) * d).
//
// Design for gfx950 (measured: LDS reads ~128 B/clk/CU, fp16 MFMA ~2.2 PF):
//   * A workgroup of 4 waves owns a 256 x 128 output tile; wave (wm, wn) owns
//     rows 128 wm .. +128 and columns 64 wn .. +64, i.e. 4 x 2 blocks of
//     32 x 32 accumulators (128 fp32 per lane).  K advances 64 (two Q4_0
//     blocks) per step.
//   * X (fp16) goes through LDS, double-buffered with an XOR swizzle of the
//     16-byte chunks of each row (conflict-free ds_read_b128 / ds_write_b128),
//     one barrier per K step; the next step's X loads are in flight while the
//     current step's matrix instructions run.
//   * W never touches LDS: each wave's 64 columns are exactly one 64-row tile
//     of the packed layout, and the MFMA B operand of lane l is 8 consecutive
//     weights of column l % 32, i.e. 8 code bytes of one block.  The low
//     nibbles of bytes 8h .. 8h+7 are elements 8h .. 8h+7 and the high nibbles
//     elements 16+8h .. 16+8h+7 (GGUF order), so one 8-byte load per lane
//     gives the B fragments of both 16-deep halves of the block.  v_perm_b32
//     places each nibble under the fp16 exponent 2^10, v_pk_add_f16 removes
//     1032 (exact q - 8) and v_pk_mul_f16 applies d with one rounding.  The
//     loads for the next step are issued a step ahead.
//   * Few output tiles (the 2048 x 11008 down projection has 32) split K
//     across workgroups: each slice writes its partial tile to the caller's
//     workspace and a second kernel adds the slices in order (deterministic).
//   * Workgroups that read the same weights (same N tile, different M tile)
//     are placed on the same XCD so the second read hits that XCD's L2.
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
constexpr int kThreads = 256;
constexpr int kRowBytes = 128;                 // one LDS row of X: 64 halves (two blocks)
// One ring slot: X (256 rows x 128 B), then the codes of two blocks of two
// packed tiles (4 x 1 KB), then their scales (4 x 256 B: a 2-byte load to
// LDS fills one dword per lane, zero-extended).
constexpr int kWOff = BM * kRowBytes;
constexpr int kSOff = kWOff + 4 * 1024;
constexpr int kSlotBytes = kSOff + 4 * 256;    // 37,888 B
constexpr int kStages = 4;                     // ring depth: loads run three steps ahead
constexpr int kLoadsPerStep = 10;              // per wave: 8 X, 1 code, 1 scale
constexpr int kLdsBytes = kStages * kSlotBytes;   // 151,552 B of the 160 KB
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
    int32_t tiles_m, tiles_n, S, us;   // us: blocks per K slice (even)
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

// B fragments of one block for this lane: 8 code bytes (bytes 8h .. 8h+7 of
// the block), fp16 scale d.  lo: elements 8h .. 8h+7, hi: 16+8h .. 16+8h+7.
__device__ __forceinline__ void dequant_frag(u32x2 c, uint16_t d, half8_t& lo, half8_t& hi) {
    const _Float16 dh = __builtin_bit_cast(_Float16, d);
    const half2_t dd = {dh, dh};
    const uint32_t l0 = c.x & 0x0F0F0F0Fu, l1 = c.y & 0x0F0F0F0Fu;
    const uint32_t h0 = (c.x >> 4) & 0x0F0F0F0Fu, h1 = (c.y >> 4) & 0x0F0F0F0Fu;
    const u32x4 a = {w2(l0, 0x04010400u, dd), w2(l0, 0x04030402u, dd), w2(l1, 0x04010400u, dd),
                     w2(l1, 0x04030402u, dd)};
    const u32x4 b = {w2(h0, 0x04010400u, dd), w2(h0, 0x04030402u, dd), w2(h1, 0x04010400u, dd),
                     w2(h1, 0x04030402u, dd)};
    lo = __builtin_bit_cast(half8_t, a);
    hi = __builtin_bit_cast(half8_t, b);
}

// LDS byte offset of 16-byte chunk `chunk` of X row `row`.  The chunk index
// is XORed with bits 1-3 of the row: the 16 lanes that one LDS cycle serves
// (64 banks of 4 bytes) then read or write 16 distinct (row parity, chunk)
// slots, so fragment reads (16 rows, one chunk) and row stores (2 rows,
// 8 chunks) are both free of bank conflicts.
__device__ __forceinline__ uint32_t lds_off(int row, int chunk) {
    return uint32_t(row) * kRowBytes + uint32_t((chunk ^ ((row >> 1) & 7)) * 16);
}

// Workgroup barrier that orders LDS accesses (a compiler memory barrier) but
// adds no wait of its own: __syncthreads() would also wait for every
// outstanding global load, including the copy-engine loads of later steps
// that are meant to stay in flight across it.  Callers wait explicitly for
// the loads they need first.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS accesses done
    asm volatile("s_barrier" ::: "memory");
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// of this wave are outstanding (lgkm and exp counters left unconstrained).
constexpr int vmcnt_imm(int n) { return (n & 15) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14); }

__global__ __launch_bounds__(kThreads, 1) void gemm_q4_0_kernel(const GemmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];   // kStages x kSlotBytes

    // Work item: M tile fastest, then N tile, then K slice.
    int L = blockIdx.x;
    if (a.remap) L = (L % 8) * int(gridDim.x / 8) + L / 8;
    const int tm = L % a.tiles_m;
    const int rest = L / a.tiles_m;
    const int tn = rest % a.tiles_n;
    const int ks = rest / a.tiles_n;
    const int m0 = tm * BM;
    const int u0 = ks * a.us;
    const int u1 = min(a.nu, u0 + a.us);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5;
    const int tiles_b = (a.N + kTileRows - 1) / kTileRows;

    // ---- copy engine: one step = 64 columns of X (256 rows) + two blocks of
    // W for the workgroup's two packed tiles, all straight into LDS with
    // global_load_lds (no registers).  Per step each wave issues exactly
    // kLoadsPerStep loads: 8 X row groups, 1 block of codes, 1 of scales.
    //   X: wave w, load i covers rows 8 (8w + i) .. +8.  Lane s fills LDS
    //      slot bytes s * 16 of that 1 KB run, i.e. row 8 (8w + i) + s / 8,
    //      physical chunk s % 8, which holds logical chunk
    //      (s % 8) ^ ((row >> 1) & 7) of the swizzled layout (lds_off).
    //   W: wave w loads block (w & 1) of packed tile 2 tn + (w >> 1): lane s
    //      takes row s (clamped into the tile) of that block's 1 KB run, and
    //      its scale (which lands in the low half of LDS dword s).
    uint32_t xo[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = 8 * (8 * wave + i) + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        xo[i] = uint32_t(min(m0 + row, a.M - 1)) * uint32_t(a.K) * 2u + uint32_t(c) * 16u;
    }
    const int lt = wave >> 1, lq = wave & 1;                 // tile, block this wave loads
    const int ltb = min(tn * 2 + lt, tiles_b - 1);
    const int lnr = min(kTileRows, a.N - ltb * kTileRows);
    const uint8_t* lcode = a.codes + size_t(ltb) * kTileRows * size_t(a.nu) * 16;
    const uint16_t* lscale = a.scales + size_t(ltb) * kTileRows * size_t(a.nu);
    const uint32_t lrow = uint32_t(min(lane, lnr - 1));
    auto issue = [&](int st) {   // loads of step st into slot st % kStages
        uint8_t* slot = lds + (st % kStages) * kSlotBytes;
        const int ub = u0 + 2 * st;
        const uint8_t* xb = reinterpret_cast<const uint8_t*>(a.X) + size_t(ub) * 64;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(xb + xo[i]),
                (__attribute__((address_space(3))) void*)(slot + (8 * wave + i) * 1024), 16, 0, 0);
        const size_t e = size_t(ub + lq) * size_t(lnr) + lrow;
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(lcode + e * 16),
            (__attribute__((address_space(3))) void*)(slot + kWOff + (lt * 2 + lq) * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(lscale + e),
            (__attribute__((address_space(3))) void*)(slot + kSOff + (lt * 2 + lq) * 256), 2, 0, 0);
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // A fragments of sub-step s (16 deep) of the step whose X is at `xs`.
    auto a_frags = [&](const uint8_t* xs, int s, half8_t (&af)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = wm * 128 + i * 32 + (lane & 31);
            af[i] = *reinterpret_cast<const half8_t*>(xs + lds_off(row, 2 * s + h));
        }
    };
    auto mfma8 = [&](const half8_t (&af)[4], const half8_t (&b)[2]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], b[j], acc[i][j], 0, 0, 0);
    };
    // Sub-steps 0-3 of one step; A fragments are read one sub-step ahead.
    auto mfma_sub = [&](const uint8_t* xs, int s, const half8_t (&b)[2]) {
        half8_t af[4];
        a_frags(xs, s, af);
        mfma8(af, b);
    };
    // B fragments of block q of the step in `slot` (this wave's tile wn).
    auto b_frags = [&](const uint8_t* slot, int q, half8_t (&lo)[2], half8_t (&hi)[2]) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = 32 * j + (lane & 31);
            const u32x2 c = *reinterpret_cast<const u32x2*>(slot + kWOff + (wn * 2 + q) * 1024 + r * 16 + 8 * h);
            const uint16_t d = *reinterpret_cast<const uint16_t*>(slot + kSOff + (wn * 2 + q) * 256 + r * 4);
            dequant_frag(c, d, lo[j], hi[j]);
        }
    };

    // Full steps (two blocks) run through the ring; a slice with an odd
    // block count ends with a one-block tail step after the loop.  At the top
    // of step st the loads of steps st and st + 1 have landed (the weights of
    // step st + 1 are unpacked while step st's second block multiplies),
    // step st + 2 may be in flight and step st + 3 is issued.  Near the end
    // the issue index is clamped to the last step: the copy lands in a slot
    // nobody reads any more, and every step issues the same number of loads,
    // so the wait count is a constant and the loop body is one basic block.
    const int nfull = (u1 - u0) >> 1;
    half8_t b0lo[2], b0hi[2];   // block 0 of the current step, unpacked ahead
    if (nfull > 0) {
#pragma unroll
        for (int p = 0; p < kStages - 1; ++p) issue(min(p, nfull - 1));
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kLoadsPerStep));
        lds_barrier();
        b_frags(lds, 0, b0lo, b0hi);
    }
    for (int st = 0; st < nfull; ++st) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadsPerStep));
        lds_barrier();   // also: every wave is done with the slot refilled next
        issue(min(st + kStages - 1, nfull - 1));
        const uint8_t* slot = lds + (st % kStages) * kSlotBytes;
        const uint8_t* next = lds + ((st + 1) % kStages) * kSlotBytes;
        // All A fragments of the step are read up front (one LDS latency per
        // step instead of one per sub-step), block 1 is unpacked while they
        // arrive, and the next step's block 0 is unpacked under the matrix
        // instructions of this step's block 1.
        half8_t af[4][4];
#pragma unroll
        for (int s = 0; s < 4; ++s) a_frags(slot, s, af[s]);
        half8_t b1lo[2], b1hi[2];
        b_frags(slot, 1, b1lo, b1hi);
        mfma8(af[0], b0lo);
        mfma8(af[1], b0hi);
        b_frags(next, 0, b0lo, b0hi);   // past the last step: unused data of a dead slot
        mfma8(af[2], b1lo);
        mfma8(af[3], b1hi);
    }
    if ((u1 - u0) & 1) {
        // One-block tail through registers into the slot after the last step
        // (its last reads ended before a barrier already passed): columns
        // 32 ub .. 32 ub + 31 in chunks 0-3; chunks 4-7 are never read (only
        // sub-steps 0 and 1 run).
        const int ub = u1 - 1;
        uint8_t* slot = lds + (nfull % kStages) * kSlotBytes;
        const int xr = tid >> 3, xc = tid & 3;
        const _Float16* xb = a.X + size_t(ub) * 32 + xc * 8;
        if ((tid & 7) < 4) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = xr + 32 * i;
                *reinterpret_cast<u32x4*>(slot + lds_off(row, xc)) =
                    *reinterpret_cast<const u32x4*>(xb + size_t(min(m0 + row, a.M - 1)) * a.K);
            }
        }
        half8_t blo[2], bhi[2];
        const int tb = min(tn * 2 + wn, tiles_b - 1);
        const int nr = min(kTileRows, a.N - tb * kTileRows);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const size_t e = size_t(ub) * size_t(nr) + size_t(min(32 * j + (lane & 31), nr - 1));
            const u32x2 c = *reinterpret_cast<const u32x2*>(a.codes + size_t(tb) * kTileRows * size_t(a.nu) * 16 + e * 16 + 8 * h);
            const uint16_t d = a.scales[size_t(tb) * kTileRows * size_t(a.nu) + e];
            dequant_frag(c, d, blo[j], bhi[j]);
        }
        __syncthreads();
        mfma_sub(slot, 0, blo);
        mfma_sub(slot, 1, bhi);
    }

    // Epilogue: the 256 x 128 tile goes through LDS (the ring is free now)
    // so that global stores are whole 512-byte rows, 16 bytes per lane.
    // 32x32 accumulator layout: register r of lane l is row 8 (r / 4) +
    // 4 (l / 32) + r % 4, column l % 32.  Row pitch 136 floats: the two half
    // waves (rows 4 apart) write disjoint banks.
    constexpr int kCPitch = BN + 8;
    __syncthreads();
    float* cst = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * 128 + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                const int col = wn * 64 + j * 32 + (lane & 31);
                cst[row * kCPitch + col] = acc[i][j][r];
            }
    __syncthreads();
    float* out = a.out + size_t(ks) * size_t(a.M) * size_t(a.N);
    const int n0 = tn * BN;
    const int col = (tid & 31) * 4;
    const bool full = m0 + BM <= a.M && n0 + BN <= a.N && (a.N & 3) == 0;
#pragma unroll 4
    for (int k = 0; k < BM / 8; ++k) {
        const int row = (tid >> 5) + 8 * k;
        const f32x4 v = *reinterpret_cast<const f32x4*>(cst + row * kCPitch + col);
        const int m = m0 + row;
        if (full) {
            *reinterpret_cast<f32x4*>(out + size_t(m) * size_t(a.N) + n0 + col) = v;
        } else if (m < a.M) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n0 + col + e < a.N) out[size_t(m) * size_t(a.N) + n0 + col + e] = v[e];
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
    S = std::min(S, std::max(1, nu / 16));   // at least 16 blocks (8 steps) per slice
    int us = (nu + S - 1) / S;
    us += us & 1;                            // whole steps of two blocks
    p.us = us;
    p.S = (nu + us - 1) / us;                // no empty slice
    return p;
}

}  // namespace

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const Plan p = plan_gemm(M, N, K);
    return p.S > 1 ? size_t(p.S) * size_t(M) * size_t(N) * sizeof(float) : 0;
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
    const size_t mn = size_t(M) * size_t(N);
    const size_t blocks = (mn + 1023) / 1024;
    hipLaunchKernelGGL(splitk_reduce, dim3(unsigned(blocks)), dim3(256), 0, stream,
                       static_cast<const float*>(ws), Y, mn, p.S);
    return hipGetLastError();
}

}  // namespace lq
