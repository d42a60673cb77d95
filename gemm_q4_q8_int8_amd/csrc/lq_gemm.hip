// Prefill GEMM for Q4_0, Q8_0 and int8 block-64 weights:
// Y[M x N] = X[M x K] * W[N x K]^T.
//
// Prefill is compute-bound ("oxinfer" page, "Performance"), and the GPU
// kernels the page describes dequantize the weight tile on chip before the
// dense contraction ("Platforms and accelerators": weights dequantized in
// threadgroup memory).  On gfx950 the dense step is the fp16 matrix-core
// instruction v_mfma_f32_32x32x16_f16 (fp32 accumulate).  Q4_0 and Q8_0
// weights are rounded once to fp16: RN_fp16((q - 8) * d), RN_fp16(c * d).
// int8 block-64 scales are fp32, not fp16 values: the B tile holds the exact
// codes, the two steps of a 64-element unit accumulate into a second set of
// accumulators, and the unit's scale multiplies that block sum in fp32.
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
//   * The epilogue stores straight from the accumulators (128-byte row
//     segments).
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
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kXRowBytes = 64;

// Layout of one workgroup's LDS for format FMT (Q4_0 or Q8_0) and NT packed
// 64-row weight tiles (a 256 x 64 NT output tile).  One ring slot: X (256
// rows x 64 B), the codes of one block of the NT packed tiles (P = 1 or 2
// parts of 1 KB each per tile, in packed order), their scales (NT x 256 B: a
// 2-byte load to LDS fills one dword per lane, zero-extended), and 256 B that
// absorb the extra loads of waves with nothing else to copy.  Behind the
// ring: three fp16 B tiles (64 NT columns x 32).  Each wave issues two X
// loads and kOthers code / scale / spare loads per step.
template <int FMT, int NT>
struct Cfg {
    static constexpr int P = FMT == kQ4_0 ? 1 : 2;                // 16-byte code parts per row per step
    static constexpr int SB = scale_bytes(FMT);
    static constexpr int SPS = unit_elems(FMT) / 32;              // steps per scale block
    static constexpr int BN = 64 * NT;
    static constexpr int kStages = (P == 2 && NT == 3) ? 5 : 6;   // copies run kStages - 2 steps ahead
    static constexpr int kOthers = (NT * P + NT + kWaves - 1) / kWaves;
    static constexpr int kLoadsPerStep = 2 + kOthers;
    static constexpr int kWOff = BM * kXRowBytes;                 // 16,384
    static constexpr int kSOff = kWOff + NT * P * 1024;
    static constexpr int kDummyOff = kSOff + NT * 256;
    static constexpr int kSlotBytes = kDummyOff + 256;
    static constexpr int kBTileBytes = BN * 64;
    static constexpr int kBOff = kStages * kSlotBytes;
    static constexpr int kLdsBytes = kBOff + 3 * kBTileBytes;     // <= 159,744
    static_assert(kLdsBytes <= 160 * 1024, "LDS");
    static_assert(kStages >= 5, "the unpack needs step st + 2 landed");
    static_assert(!fp32_scale(FMT) || NT == 2, "fp32-scale formats keep a second accumulator set");
};

// Output tiles below which K is split across workgroups, and the workgroups
// a split aims for.
constexpr int kSplitBelowTiles = 128;
constexpr int kSplitTargetWgs = 256;

// One weight matrix of a launch.  Every matrix of a launch shares X, M and
// K; its workgroups are wg0 .. wg0 + tiles_m * tiles_n * S - 1.
struct GemmMat {
    const uint8_t* codes;     // code plane (tiled layout)
    const uint8_t* scales;    // scale plane (tiled layout; fp16, or fp32 for int8 block-64)
    float* out;               // Y (S == 1) or S partial M x N slices
    int32_t N, tiles_n, wg0, pad;
};

struct GemmArgs {
    int32_t wg0[kMaxGemmGroup];   // mat[i].wg0, INT32_MAX past count (find_matrix)
    GemmMat mat[kMaxGemmGroup];
    const _Float16* X;        // M x K row-major
    int32_t count;            // matrices
    int32_t M, K, nu;         // nu = K / 32 (steps)
    int32_t tiles_m, S, us;   // us: blocks per K slice
    int32_t remap;            // 1: XCD-aware workgroup order
};

__device__ __forceinline__ uint32_t bits(half2_t h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ half2_t as_half2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// Two fp16 weights RN_fp16((q - 8) * d) from two nibbles (bytes `sel` of v).
__device__ __forceinline__ uint32_t w2(uint32_t v, uint32_t sel, half2_t dd) {
    const half2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
    return bits((as_half2(__builtin_amdgcn_perm(0x64646464u, v, sel)) - off) * dd);
}

// Two fp16 weights RN_fp16(c * d) from two sign-flipped int8 codes (bytes
// `sel` of v): under 0x64 a byte u is the fp16 value 1024 + u, and
// u - 128 = c.
__device__ __forceinline__ uint32_t w8(uint32_t v, uint32_t sel, half2_t dd) {
    const half2_t off = {(_Float16)1152.0f, (_Float16)1152.0f};
    return bits((as_half2(__builtin_amdgcn_perm(0x64646464u, v, sel)) - off) * dd);
}

// Two exact fp16 int8 codes from two sign-flipped codes (bytes `sel` of v).
__device__ __forceinline__ uint32_t wi8(uint32_t v, uint32_t sel) {
    const half2_t off = {(_Float16)1152.0f, (_Float16)1152.0f};
    return bits(as_half2(__builtin_amdgcn_perm(0x64646464u, v, sel)) - off);
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

template <int FMT, int NT>
__global__ __launch_bounds__(kThreads, 1) void gemm_tile_kernel(const GemmArgs a) {
    using C = Cfg<FMT, NT>;
    constexpr int P = C::P;
    constexpr int kStages = C::kStages;
    constexpr int kLoadsPerStep = C::kLoadsPerStep;
    constexpr int BN = C::BN;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    // Work item: matrix, then (inside it) M tile fastest, then N tile, then
    // K slice.
    int L = blockIdx.x;
    if (a.remap) L = (L % 8) * int(gridDim.x / 8) + L / 8;
    const GemmMat& G = a.mat[find_matrix(a.wg0, L)];
    const int local = L - G.wg0;
    const int rest = int(uint32_t(local) / uint32_t(a.tiles_m));
    const int tm = local - rest * a.tiles_m;
    const int ks = int(uint32_t(rest) / uint32_t(G.tiles_n));
    const int tn = rest - ks * G.tiles_n;
    const int m0 = tm * BM;
    const int u0 = ks * a.us;
    const int nst = min(a.nu, u0 + a.us) - u0;   // steps (blocks) of this slice

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5;
    const int tiles_b = (G.N + kTileRows - 1) / kTileRows;

    // ---- copy ring.  Per step each wave issues kLoadsPerStep loads:
    //   X: wave w covers rows 32 w .. +32 in two 1 KB loads; lane s of load
    //      i fills row 32 w + 16 i + s / 4, physical chunk s % 4, i.e.
    //      logical chunk (s % 4) ^ ((row >> 2) & 3).
    //   kOthers more, numbered q = w + 8 k: q < NT P: part q % P of the
    //      block's codes of packed tile NT tn + q / P (lane s: row s, clamped
    //      into the tile); then NT scale loads; the rest a spare load of
    //      scales into the slot's dummy area (keeps the per-wave count
    //      uniform for the wait).
    // Byte offsets into X are 64-bit: X may exceed 4 GiB (M K 2 bytes).
    size_t xo[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = 32 * wave + 16 * i + (lane >> 2);
        const int c = (lane & 3) ^ ((row >> 2) & 3);
        xo[i] = size_t(min(m0 + row, a.M - 1)) * size_t(a.K) * 2u + size_t(c) * 16u;
    }
    constexpr int kOthers = C::kOthers;
    const uint8_t* osrc[kOthers];   // per-lane source of the step-0 block
    uint32_t ostep[kOthers];        // source bytes per step (per scale block for scales)
    uint32_t odst[kOthers];         // LDS offset inside the slot
    int osize[kOthers];             // 16 (codes) or the scale size
    int oshift[kOthers];            // step -> source block: st >> oshift
#pragma unroll
    for (int k = 0; k < kOthers; ++k) {
        const int q = wave + kWaves * k;
        const bool code = q < NT * P;
        const int t = code ? q / P : (q < NT * P + NT ? q - NT * P : 0);
        const int ltb = min(tn * NT + t, tiles_b - 1);
        const int lnr = min(kTileRows, G.N - ltb * kTileRows);
        const uint32_t lrow = uint32_t(min(lane, lnr - 1));
        if (code) {
            osrc[k] = G.codes + size_t(ltb) * kTileRows * size_t(a.nu) * P * 16 +
                      (size_t(u0) * P + size_t(q % P)) * size_t(lnr) * 16 + lrow * 16;
            ostep[k] = uint32_t(P * lnr * 16);
            odst[k] = uint32_t(C::kWOff + q * 1024);
            osize[k] = 16;
            oshift[k] = 0;
        } else {
            // One scale per row and scale block (SPS steps); both steps of an
            // int8 block-64 unit copy its scales.
            const size_t blocks = size_t(a.nu) / C::SPS;
            osrc[k] = G.scales + (size_t(ltb) * kTileRows * blocks + size_t(u0 / C::SPS) * lnr + lrow) * C::SB;
            ostep[k] = uint32_t(lnr * C::SB);
            odst[k] = uint32_t(q < NT * P + NT ? C::kSOff + t * 256 : C::kDummyOff);
            osize[k] = C::SB;
            oshift[k] = C::SPS == 2 ? 1 : 0;
        }
    }
    auto issue = [&](int st) {   // loads of step st into slot st % kStages
        uint8_t* slot = lds + (st % kStages) * C::kSlotBytes;
        const uint8_t* xb = reinterpret_cast<const uint8_t*>(a.X) + size_t(u0 + st) * 64;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(xb + xo[i]),
                (__attribute__((address_space(3))) void*)(slot + (2 * wave + i) * 1024), 16, 0, 0);
#pragma unroll
        for (int k = 0; k < kOthers; ++k) {
            const auto* src =
                (const __attribute__((address_space(1))) void*)(osrc[k] + size_t(st >> oshift[k]) * ostep[k]);
            auto* dst = (__attribute__((address_space(3))) void*)(slot + odst[k]);
            // The copy size must be an immediate: the 16-byte (codes) or
            // scale-size form, chosen per wave.
            if (osize[k] == 16) __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
            else __builtin_amdgcn_global_load_lds(src, dst, C::SB, 0, 0);
        }
    };

    // ---- unpack: task t turns 8 weights of column n = t / 4 into one
    // 16-byte chunk of the fp16 B tile, elements 8p .. 8p + 7 of the block
    // (p = t % 4), RN_fp16(w) each.  Q4_0: the low (p < 2) or high (p >= 2)
    // nibbles of code bytes 8 (p % 2) .. 8 (p % 2) + 7 (GGUF order): under
    // fp16 exponent 2^10 minus 1032 is q - 8 exactly.  Q8_0: code bytes
    // 8p .. 8p + 7, sign bit flipped and placed under 0x64: minus 1152 is the
    // int8 code exactly.  Then one fp16 multiply by d.  There are 4 BN
    // tasks: thread t takes task t, and for NT = 3 also task 512 + t % 256
    // (waves 4-7 repeat the tasks of waves 0-3, writing the same bytes): no
    // branch, so the compiler can interleave the unpacking with the matrix
    // instructions.
    constexpr int kTasks = NT == 2 ? 1 : 2;
    static_assert(NT == 2 || NT == 3, "task split");
    uint32_t uc_off[kTasks], us_off[kTasks], ub_off[kTasks];
    int ush[kTasks];
#pragma unroll
    for (int q = 0; q < kTasks; ++q) {
        const int t = q == 0 ? tid : kThreads + (tid & 255);
        const int un = t >> 2, up = t & 3;
        if constexpr (P == 1)
            uc_off[q] = uint32_t(C::kWOff + (un >> 6) * 1024 + (un & 63) * 16 + 8 * (up & 1));
        else
            uc_off[q] = uint32_t(C::kWOff + ((un >> 6) * 2 + (up >> 1)) * 1024 + (un & 63) * 16 + 8 * (up & 1));
        us_off[q] = uint32_t(C::kSOff + (un >> 6) * 256 + (un & 63) * 4);
        ub_off[q] = sw_off(un, up);
        ush[q] = (up >> 1) * 4;
    }
    auto unpack = [&](const uint8_t* slot, uint8_t* btile) {
#pragma unroll
        for (int q = 0; q < kTasks; ++q) {
            const u32x2 c = *reinterpret_cast<const u32x2*>(slot + uc_off[q]);
            u32x4 v;
            if constexpr (fp32_scale(FMT)) {
                // Exact codes; the fp32 scale multiplies the block sums.
                const uint32_t b0 = c.x ^ 0x80808080u, b1 = c.y ^ 0x80808080u;
                v = u32x4{wi8(b0, 0x04010400u), wi8(b0, 0x04030402u), wi8(b1, 0x04010400u), wi8(b1, 0x04030402u)};
                *reinterpret_cast<u32x4*>(btile + ub_off[q]) = v;
                continue;
            }
            const uint16_t d = *reinterpret_cast<const uint16_t*>(slot + us_off[q]);
            const _Float16 dh = __builtin_bit_cast(_Float16, d);
            const half2_t dd = {dh, dh};
            if constexpr (P == 1) {
                const uint32_t n0 = (c.x >> ush[q]) & 0x0F0F0F0Fu, n1 = (c.y >> ush[q]) & 0x0F0F0F0Fu;
                v = u32x4{w2(n0, 0x04010400u, dd), w2(n0, 0x04030402u, dd), w2(n1, 0x04010400u, dd),
                          w2(n1, 0x04030402u, dd)};
            } else {
                const uint32_t b0 = c.x ^ 0x80808080u, b1 = c.y ^ 0x80808080u;
                v = u32x4{w8(b0, 0x04010400u, dd), w8(b0, 0x04030402u, dd), w8(b1, 0x04010400u, dd),
                          w8(b1, 0x04030402u, dd)};
            }
            *reinterpret_cast<u32x4*>(btile + ub_off[q]) = v;
        }
    };

    f32x16 acc[2][NT];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // ---- main loop, software-pipelined over three steps: at step st the
    // matrix instructions of step st run on fragments read during step
    // st - 1, the fragments of step st + 1 are read, and the weights of step
    // st + 2 are unpacked (B tiles are triple-buffered), so LDS latency and
    // unpacking overlap the matrix instructions instead of following a
    // barrier.  Copies run kStages - 3 steps ahead of the unpacking: at the
    // top of step st the loads of steps up to st + 2 have landed, those up to
    // st + kStages - 2 may be in flight, and st + kStages - 1 is issued
    // (clamped to the last step: past the end the copy lands in a slot nobody
    // reads, so every step issues the same number of loads and the wait
    // count is a constant).
    auto slot_of = [&](int st) { return lds + (st % kStages) * C::kSlotBytes; };
    auto btile_of = [&](int st) { return lds + C::kBOff + (st % 3) * C::kBTileBytes; };
    // Fragment offsets of this lane: A rows wm 64 + 32 i + lane % 32, B
    // columns wn 32 NT + 32 j + lane % 32, chunk 2 s + h.  Blocks 32 rows
    // apart keep the row's swizzle bits, so block i (j) is 2 KB i (j) further:
    // an immediate offset of the LDS read.
    const uint32_t a_off[2] = {sw_off(wm * 64 + (lane & 31), h), sw_off(wm * 64 + (lane & 31), 2 + h)};
    const uint32_t b_off[2] = {sw_off(wn * 32 * NT + (lane & 31), h), sw_off(wn * 32 * NT + (lane & 31), 2 + h)};
    half8_t af[2][2], bf[2][NT];   // [sub-step][block] of the next step to multiply
    auto read_frags = [&](int st) {
        const uint8_t* slot = slot_of(st);
        const uint8_t* bt = btile_of(st);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int i = 0; i < 2; ++i) af[s][i] = *reinterpret_cast<const half8_t*>(slot + a_off[s] + i * 2048);
#pragma unroll
            for (int j = 0; j < NT; ++j) bf[s][j] = *reinterpret_cast<const half8_t*>(bt + b_off[s] + j * 2048);
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
    auto step = [&](int st, f32x16 (&dst)[2][NT]) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((kStages - 4) * kLoadsPerStep));   // step st + 2 landed
        lds_barrier();
        issue(min(st + kStages - 1, nst - 1));
        unpack(slot_of(st + 2), btile_of(st + 2));   // past the last step: unused data
        half8_t a0[2][2], b0[2][NT];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int i = 0; i < 2; ++i) a0[s][i] = af[s][i];
#pragma unroll
            for (int j = 0; j < NT; ++j) b0[s][j] = bf[s][j];
        }
        read_frags(st + 1);                          // past the last step: unused data
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    dst[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[s][i], b0[s][j], dst[i][j], 0, 0, 0);
    };
    if constexpr (fp32_scale(FMT)) {
        // The SPS steps of a unit (2 for 64-element units, 1 for 32)
        // accumulate exact-code products into blk; the unit's fp32 scale of
        // column n (this lane's column in every accumulator register) then
        // multiplies the block sum, read from the unit's last step's slot
        // (every step copies its unit's scales).  Slices hold whole units,
        // so nst is a multiple of SPS.
        constexpr int SPS = C::SPS;
        const uint32_t s_off[NT] = {uint32_t(C::kSOff + wn * 256 + (lane & 31) * 4),
                                    uint32_t(C::kSOff + wn * 256 + (32 + (lane & 31)) * 4)};
        for (int st = 0; st < nst; st += SPS) {
            f32x16 blk[2][NT];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) blk[i][j][r] = 0.0f;
#pragma unroll
            for (int q = 0; q < SPS; ++q) step(st + q, blk);
            const uint8_t* slot = slot_of(st + SPS - 1);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const float sc = *reinterpret_cast<const float*>(slot + s_off[j]);
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    acc[i][j] = __builtin_elementwise_fma(f32x16(sc), blk[i][j], acc[i][j]);
            }
        }
    } else {
        for (int st = 0; st < nst; ++st) step(st, acc);
    }

    // ---- epilogue: straight from the accumulators.  32x32 accumulator
    // layout: register r of lane l is row 8 (r / 4) + 4 (l / 32) + r % 4,
    // column l % 32, so each store writes two 128-byte row segments.  (Staging
    // the tile through LDS for whole-row 16-byte stores took two barriers and
    // was 1.4 us slower on the 2048 x 11008 gate + up launch at M = 512.)
    float* out = G.out + size_t(ks) * size_t(a.M) * size_t(G.N);
    const int n0 = tn * BN;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int col = n0 + wn * 32 * NT + j * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 64 + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                if (row < a.M && col < G.N) out[size_t(row) * size_t(G.N) + col] = acc[i][j][r];
            }
        }
}

// ------------------------------------------------------------------------
// Wave-fragment GEMM for the fp16-scale formats (Q4_0, Q8_0).
//
// A workgroup of 4 waves, one per SIMD, owns a (64 MI) x (64 NJ) output tile;
// wave (wm, wn) owns rows 32 MI wm .. +32 MI and columns 32 NJ wn .. +32 NJ,
// MI x NJ blocks of 32 x 32 fp32 accumulators (accumulation registers).  The
// copy ring (global_load_lds, straight to LDS) carries the step's X tile and
// the raw codes and scales of the workgroup's NJ packed 64-row tiles, D - 2
// steps ahead of use.  Each wave decodes the weight fragments it multiplies
// itself, in registers, from the raw codes in LDS: lane (c, h) of block j
// takes bytes 8h .. 8h + 7 of column c's block, whose low nibbles (Q4_0) or
// first code part (Q8_0) are elements 8h .. 8h + 7 of the first 16-element
// half of the block and whose high nibbles / second part are elements
// 16 + 8h .. of the second, exactly the B operand layout of
// v_mfma_f32_32x32x16_f16.  No decoded tile is written back to LDS, and the
// one barrier per step only guards the ring.  A wave's vector work (decode,
// fragment reads, copy issue) runs while its own matrix instructions execute
// (measured: a wave per SIMD issuing 24 of them and ~130 decode-like vector
// ops per step runs at the matrix-only rate), so the step costs its matrix
// time: the MFMAs of step st use fragments prepared during step st - 1.

template <int FMT, int MI, int NJ>
struct WCfg {
    static constexpr int P = FMT == kQ4_0 ? 1 : 2;
    static constexpr int BM = 64 * MI;
    static constexpr int BN = 64 * NJ;
    static constexpr int NT = NJ;                          // packed 64-row tiles per workgroup
    static constexpr int kXBytes = BM * kXRowBytes;
    static constexpr int kWOff = kXBytes;
    static constexpr int kSOff = kWOff + NT * P * 1024;
    static constexpr int kSlotBytes = kSOff + NT * 256;
    // Behind the ring: where the copies of waves with nothing to copy land
    // (1 KB for a code copy, 256 B for a scale copy); nothing reads it.
    static constexpr int kDummyBytes = 1024 + 256;
    static constexpr int kStages =
        (160 * 1024 - kDummyBytes) / kSlotBytes > 8 ? 8 : (160 * 1024 - kDummyBytes) / kSlotBytes;
    static constexpr int kDummyOff = kStages * kSlotBytes;
    static constexpr int kLdsBytes = kDummyOff + kDummyBytes;
    static constexpr int kXLoads = BM / 16;                // 1 KB copies of X per step
    static constexpr int kXPerWave = kXLoads / 4;
    static constexpr int kCodePerWave = (NT * P + 3) / 4;  // 16-byte code copies (wave w: parts w + 4 k)
    static constexpr int kScalePerWave = (NT + 3) / 4;     // 2-byte scale copies
    static constexpr int kLoadsPerStep = kXPerWave + kCodePerWave + kScalePerWave;
    static_assert(kXLoads % 4 == 0, "X copies split evenly");
    static_assert(kStages >= 4, "ring depth");
    static_assert((kStages - 2) * kLoadsPerStep <= 63, "vmcnt range");
    static_assert(kLdsBytes <= 160 * 1024, "LDS");
};

template <int FMT, int MI, int NJ>
__global__ __launch_bounds__(256, 1) void gemm_wave_kernel(const GemmArgs a) {
    using C = WCfg<FMT, MI, NJ>;
    constexpr int P = C::P;
    constexpr int D = C::kStages;
    constexpr int L = C::kLoadsPerStep;
    constexpr int NT = C::NT;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    int Lw = blockIdx.x;
    if (a.remap) Lw = (Lw % 8) * int(gridDim.x / 8) + Lw / 8;
    const GemmMat& G = a.mat[find_matrix(a.wg0, Lw)];
    const int local = Lw - G.wg0;
    const int rest = int(uint32_t(local) / uint32_t(a.tiles_m));
    const int tm = local - rest * a.tiles_m;
    const int ks = int(uint32_t(rest) / uint32_t(G.tiles_n));
    const int tn = rest - ks * G.tiles_n;
    const int m0 = tm * C::BM;
    const int u0 = ks * a.us;
    const int nst = min(a.nu, u0 + a.us) - u0;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int c = lane & 31, h = lane >> 5;
    const int tiles_b = (G.N + kTileRows - 1) / kTileRows;

    // ---- copy ring: kXPerWave X copies (rows 16 (4 k + ... ) of the tile),
    // then kOthers code / scale / spare copies, numbered q = wave + 4 k.
    size_t xo[C::kXPerWave];
#pragma unroll
    for (int i = 0; i < C::kXPerWave; ++i) {
        const int row = 16 * (C::kXPerWave * wave + i) + (lane >> 2);
        const int ch = (lane & 3) ^ ((row >> 2) & 3);
        xo[i] = size_t(min(m0 + row, a.M - 1)) * size_t(a.K) * 2u + size_t(ch) * 16u;
    }
    // Code copy k of wave w carries part q = w + 4 k (packed tile q / P,
    // code part q % P) and scale copy k the scales of packed tile w + 4 k;
    // copies past the last real one go to the dummy area.  Every wave issues
    // the same copies of each kind, so the copy code has no branch.
    const uint8_t* csrc[C::kCodePerWave];
    uint32_t cstep[C::kCodePerWave], cdst[C::kCodePerWave];
#pragma unroll
    for (int k = 0; k < C::kCodePerWave; ++k) {
        const int q = wave + 4 * k;
        const bool real = q < NT * P;
        const int t = real ? q / P : 0;
        const int ltb = min(tn * NT + t, tiles_b - 1);
        const int lnr = min(kTileRows, G.N - ltb * kTileRows);
        const uint32_t lrow = uint32_t(min(lane, lnr - 1));
        csrc[k] = G.codes + size_t(ltb) * kTileRows * size_t(a.nu) * P * 16 +
                  (size_t(u0) * P + size_t(real ? q % P : 0)) * size_t(lnr) * 16 + lrow * 16;
        cstep[k] = uint32_t(P * lnr * 16);
        cdst[k] = real ? uint32_t(C::kWOff + q * 1024) : ~0u;
    }
    const uint8_t* ssrc[C::kScalePerWave];
    uint32_t sstep[C::kScalePerWave], sdst[C::kScalePerWave];
#pragma unroll
    for (int k = 0; k < C::kScalePerWave; ++k) {
        const int t0 = wave + 4 * k;
        const bool real = t0 < NT;
        const int t = real ? t0 : 0;
        const int ltb = min(tn * NT + t, tiles_b - 1);
        const int lnr = min(kTileRows, G.N - ltb * kTileRows);
        const uint32_t lrow = uint32_t(min(lane, lnr - 1));
        ssrc[k] = G.scales + (size_t(ltb) * kTileRows * size_t(a.nu) + size_t(u0) * lnr + lrow) * 2;
        sstep[k] = uint32_t(lnr * 2);
        sdst[k] = real ? uint32_t(C::kSOff + t * 256) : ~0u;
    }
    auto slot_of = [&](int st) { return lds + (st % D) * C::kSlotBytes; };
    // Copy n (0 .. L - 1) of step st: X copies, then code copies, then scale
    // copies (n is a compile-time index after unrolling).
    auto issue_one = [&](int st, int n) {
        uint8_t* slot = slot_of(st);
        if (n < C::kXPerWave) {
            const uint8_t* xb = reinterpret_cast<const uint8_t*>(a.X) + size_t(u0 + st) * 64;
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(xb + xo[n]),
                (__attribute__((address_space(3))) void*)(slot + (C::kXPerWave * wave + n) * 1024), 16, 0, 0);
        } else if (n < C::kXPerWave + C::kCodePerWave) {
            const int k = n - C::kXPerWave;
            uint8_t* dst = cdst[k] == ~0u ? lds + C::kDummyOff : slot + cdst[k];
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(csrc[k] + size_t(st) * cstep[k]),
                (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
        } else {
            const int k = n - C::kXPerWave - C::kCodePerWave;
            uint8_t* dst = sdst[k] == ~0u ? lds + C::kDummyOff + 1024 : slot + sdst[k];
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(ssrc[k] + size_t(st) * sstep[k]),
                (__attribute__((address_space(3))) void*)dst, 2, 0, 0);
        }
    };
    auto issue = [&](int st) {
#pragma unroll
        for (int n = 0; n < L; ++n) issue_one(st, n);
    };

    // ---- fragments.  A: lane (c, h) of block i, half s: X row
    // 32 MI wm + 32 i + c, elements 16 s + 8 h .. + 7 (chunk 2 s + h).
    // B: block j is the wave's block wn NJ + j of the workgroup's columns:
    // packed tile (wn NJ + j) / 2, rows 32 ((wn NJ + j) % 2) + c.
    uint32_t a_off[2], b_code[NJ], b_scale[NJ];
#pragma unroll
    for (int s = 0; s < 2; ++s) a_off[s] = sw_off(32 * MI * wm + c, 2 * s + h);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int bj = wn * NJ + j;
        const int rr = 32 * (bj & 1) + c;
        b_code[j] = uint32_t(C::kWOff + (bj >> 1) * P * 1024 + rr * 16 + 8 * h);
        b_scale[j] = uint32_t(C::kSOff + (bj >> 1) * 256 + rr * 4);
    }
    f32x16 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Fragments of a step: A[s][i], B[s][j] for the two 16-element halves s
    // (B as the four dwords of the 8 fp16 weights).
    struct Frags {
        half8_t a[2][MI];
        u32x4 b[2][NJ];
    };
    // Raw codes and scale of block j, and the decoded dwords: dword e of half
    // s is the weight pair (8h + 2e, 8h + 2e + 1) of that half.
    struct Raw {
        u32x2 cw[NJ][P];
        uint32_t dv[NJ];
    };
    auto read_raw = [&](const uint8_t* slot, Raw& r) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
#pragma unroll
            for (int p = 0; p < P; ++p) r.cw[j][p] = *reinterpret_cast<const u32x2*>(slot + b_code[j] + p * 1024);
            r.dv[j] = *reinterpret_cast<const uint16_t*>(slot + b_scale[j]);
        }
    };
    auto read_a = [&](const uint8_t* slot, Frags& f) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < MI; ++i) f.a[s][i] = *reinterpret_cast<const half8_t*>(slot + a_off[s] + i * 2048);
    };
    // Pair e (0..3) of half s of block j.  Q4_0: the low nibbles of the 8
    // code bytes are half 0, the high nibbles half 1; Q8_0: code part s.
    auto decode = [&](const Raw& r, int j, int s, int e) -> uint32_t {
        const _Float16 dh = __builtin_bit_cast(_Float16, uint16_t(r.dv[j]));
        const half2_t dd = {dh, dh};
        const uint32_t sel = (e & 1) ? 0x04030402u : 0x04010400u;
        if constexpr (P == 1) {
            const uint32_t w = (e & 2) ? r.cw[j][0].y : r.cw[j][0].x;
            const uint32_t n = (s ? (w >> 4) : w) & 0x0F0F0F0Fu;
            return w2(n, sel, dd);
        } else {
            const uint32_t w = ((e & 2) ? r.cw[j][s].y : r.cw[j][s].x) ^ 0x80808080u;
            return w8(w, sel, dd);
        }
    };
    auto mfma = [&](const Frags& f, int g) {
        const int s = g / (MI * NJ), i = (g / NJ) % MI, j = g % NJ;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[s][i], __builtin_bit_cast(half8_t, f.b[s][j]),
                                                           acc[i][j], 0, 0, 0);
    };

    // One step: the matrix instructions of step st on `cur`, one at a time,
    // each followed by a slice of the work for step st + 1: first the raw
    // code and scale reads, then one copy of step st + D - 1 per slice, then
    // two decoded weight pairs per slice (the A fragment reads of step st + 1
    // go behind the first of those, whose wait for the raw codes would
    // otherwise also wait for them).  This work issues while the matrix core
    // runs; sched_barrier(0) keeps the compiler from regrouping the slices.
    constexpr int kMfma = 2 * MI * NJ;
    constexpr int kPairs = 8 * NJ;
    constexpr int kFirstDec = 1 + L;
    static_assert(kFirstDec + kPairs / 2 <= kMfma, "slices");
    auto step = [&](int st, const Frags& cur, Frags& nxt) {
        // Step st + 1 has landed for every wave, and every wave is done with
        // step st - 1, whose slot the copies below may now refill.
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((D - 3) * L));
        lds_barrier();
        const uint8_t* slot = slot_of(st + 1);            // past the last step: unused data
        const int cst = min(st + D - 1, nst - 1);
        Raw raw;
#pragma unroll
        for (int g = 0; g < kMfma; ++g) {
            mfma(cur, g);
            __builtin_amdgcn_sched_barrier(0);
            if (g == 0) {
                read_raw(slot, raw);
            } else if (g < kFirstDec) {
                issue_one(cst, g - 1);
            } else if (g < kFirstDec + kPairs / 2) {
#pragma unroll
                for (int q = 2 * (g - kFirstDec); q < 2 * (g - kFirstDec) + 2; ++q) {
                    const int j = q / 8, s = (q / 4) & 1, e = q & 3;
                    nxt.b[s][j][e] = decode(raw, j, s, e);
                }
                if (g == kFirstDec) {
                    __builtin_amdgcn_sched_barrier(0);
                    read_a(slot, nxt);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    if (nst > 0) {
        Frags f0, f1;
#pragma unroll
        for (int p = 0; p < D - 1; ++p) issue(min(p, nst - 1));
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((D - 2) * L));   // step 0 landed
        lds_barrier();
        {
            Raw raw;
            read_raw(slot_of(0), raw);
            read_a(slot_of(0), f0);
#pragma unroll
            for (int q = 0; q < kPairs; ++q) f0.b[(q / 4) & 1][q / 8][q & 3] = decode(raw, q / 8, (q / 4) & 1, q & 3);
        }
        int st = 0;
        for (; st + 1 < nst; st += 2) {
            step(st, f0, f1);
            step(st + 1, f1, f0);
        }
        if (st < nst) step(st, f0, f1);
    }

    // ---- epilogue: straight from the accumulators (register r of lane l is
    // row 8 (r / 4) + 4 (l / 32) + r % 4 of the block, column l % 32).
    // A wave whose rows and columns all exist stores without checks: the row
    // part of each address is wave-uniform, the lane part fixed.
    float* out = G.out + size_t(ks) * size_t(a.M) * size_t(G.N);
    const int n0 = tn * C::BN + 32 * NJ * wn;
    const int r0 = m0 + 32 * MI * wm;
    const size_t lane_off = size_t(4 * h) * size_t(G.N) + size_t(c);
    if (r0 + 32 * MI <= a.M && n0 + 32 * NJ <= G.N) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float* rowp = out + size_t(r0 + 32 * i + 8 * (r / 4) + (r % 4)) * size_t(G.N) + (n0 + 32 * j);
                    rowp[lane_off] = acc[i][j][r];
                }
        return;
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int col = n0 + 32 * j + c;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = r0 + 32 * i + 8 * (r / 4) + 4 * h + (r % 4);
                if (row < a.M && col < G.N) out[size_t(row) * size_t(G.N) + col] = acc[i][j][r];
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

// Tile width and K split of a launch of `count` matrices that share X:
// NT packed 64-row tiles per workgroup (2 or 3) and S K slices (single
// matrices with few output tiles only).  One workgroup fits a CU's LDS, so
// the launch takes ceil(workgroups / CUs) rounds of NT x (blocks per slice)
// steps' work each.  The wide tile is taken only where it needs no K split
// and does less of that work (a fused FFN gate + up at M = 512: 232
// workgroups in one round instead of 344 in two); with a split its partial
// sums cost more than it gained (measured on the 11008 x 2048 matrix alone).
struct Plan {
    int nt, tiles_m, S, us;
    int64_t wgs;
};

// sps: steps per scale block (2 for int8 block-64: a K slice holds whole
// 64-element units).
Plan plan_for(int nt, int64_t M, const int64_t* N, int count, int64_t K, int sps) {
    Plan p;
    p.nt = nt;
    p.tiles_m = int((M + BM - 1) / BM);
    int64_t tiles = 0;
    for (int i = 0; i < count; ++i) tiles += int64_t(p.tiles_m) * ((N[i] + 64 * nt - 1) / (64 * nt));
    const int nu = int(K / 32);
    int S = 1;
    if (count == 1 && tiles < kSplitBelowTiles) S = int(std::max<int64_t>(1, kSplitTargetWgs / tiles));
    S = std::min(S, std::max(1, nu / 16));   // at least 16 blocks (steps) per slice
    const int us = (nu + S - 1) / S;
    p.us = (us + sps - 1) / sps * sps;
    p.S = (nu + p.us - 1) / p.us;            // no empty slice
    p.wgs = tiles * p.S;
    return p;
}

Plan plan_gemm(int fmt, int64_t M, const int64_t* N, int count, int64_t K, int cus) {
    if (fp32_scale(fmt)) return plan_for(2, M, N, count, K, unit_elems(fmt) / 32);
#ifdef LQ_GEMM_NT_ONLY
    return plan_for(LQ_GEMM_NT_ONLY, M, N, count, K, 1);
#endif
    const Plan p2 = plan_for(2, M, N, count, K, 1), p3 = plan_for(3, M, N, count, K, 1);
    if (p3.S > 1) return p2;
    const int64_t c = std::max(cus, 1);
    const int64_t w2 = (p2.wgs + c - 1) / c * 2 * p2.us, w3 = (p3.wgs + c - 1) / c * 3 * p3.us;
    return w3 < w2 ? p3 : p2;
}

template <int FMT, int NT>
hipError_t launch_tile(const GemmArgs& a, int64_t grid, hipStream_t stream) {
    using C = Cfg<FMT, NT>;
    // The ring needs more than the default 64 KB of dynamic LDS: raise the
    // kernel's limit once per device.
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    static std::atomic<bool> lds_ok[64];
    if (!lds_ok[dev].load(std::memory_order_acquire)) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_tile_kernel<FMT, NT>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, C::kLdsBytes);
        if (e != hipSuccess) return e;
        lds_ok[dev].store(true, std::memory_order_release);
    }
    hipLaunchKernelGGL((gemm_tile_kernel<FMT, NT>), dim3(unsigned(grid)), dim3(kThreads), C::kLdsBytes, stream, a);
    return hipGetLastError();
}

template <int FMT, int NJ>
hipError_t launch_wave(const GemmArgs& a, int64_t grid, hipStream_t stream) {
    using C = WCfg<FMT, 4, NJ>;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    static std::atomic<bool> lds_ok[64];
    if (!lds_ok[dev].load(std::memory_order_acquire)) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_wave_kernel<FMT, 4, NJ>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, C::kLdsBytes);
        if (e != hipSuccess) return e;
        lds_ok[dev].store(true, std::memory_order_release);
    }
    hipLaunchKernelGGL((gemm_wave_kernel<FMT, 4, NJ>), dim3(unsigned(grid)), dim3(256), C::kLdsBytes, stream, a);
    return hipGetLastError();
}

}  // namespace

size_t gemm_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K) {
    // Whichever tile width the launch picks (that depends on the CU count).
    size_t need = 0;
    for (int nt = 2; nt <= (fp32_scale(fmt) ? 2 : 3); ++nt) {
        const Plan p = plan_for(nt, M, &N, 1, K, unit_elems(fmt) / 32);
        if (p.S > 1) need = std::max(need, size_t(p.S) * size_t(M) * size_t(N) * sizeof(float));
    }
    return need;
}

hipError_t launch_splitk_reduce(const float* P, float* Y, size_t mn, int S, hipStream_t stream) {
    const size_t blocks = (mn + 1023) / 1024;
    hipLaunchKernelGGL(splitk_reduce, dim3(unsigned(blocks)), dim3(256), 0, stream, P, Y, mn, S);
    return hipGetLastError();
}

hipError_t launch_gemm_tile(int fmt, const void* const* W, float* const* Y, const int64_t* N, int count,
                            const void* X, int64_t M, int64_t K, void* ws, int cus, hipStream_t stream) {
    if (count < 1 || count > kMaxGemmGroup) return hipErrorInvalidValue;
    if (fmt != kQ4_0 && fmt != kQ8_0 && fmt != kI8B64 && fmt != kI8B32) return hipErrorInvalidValue;
    const Plan p = plan_gemm(fmt, M, N, count, K, cus);
    GemmArgs a = {};
    int64_t wgs = 0;
    for (int i = 0; i < count; ++i) {
        GemmMat& g = a.mat[i];
        g.codes = static_cast<const uint8_t*>(W[i]);
        g.scales = static_cast<const uint8_t*>(W[i]) + align256(code_plane_bytes(fmt, N[i], K));
        g.out = p.S > 1 ? static_cast<float*>(ws) : Y[i];
        g.N = int32_t(N[i]);
        g.tiles_n = int32_t((N[i] + 64 * p.nt - 1) / (64 * p.nt));
        g.wg0 = int32_t(wgs);
        g.pad = 0;
        wgs += int64_t(p.tiles_m) * g.tiles_n * p.S;
    }
    if (wgs > INT32_MAX) return hipErrorInvalidValue;
    fill_wg0_table(a.wg0, a.mat, count);
    a.X = static_cast<const _Float16*>(X);
    a.count = count;
    a.M = int32_t(M);
    a.K = int32_t(K);
    a.nu = int32_t(K / 32);
    a.tiles_m = p.tiles_m;
    a.S = p.S;
    a.us = p.us;
    a.remap = (wgs % 8 == 0) ? 1 : 0;
    hipError_t e;
#ifdef LQ_GEMM_TILE_ONLY
    if (fmt == kQ4_0) e = p.nt == 3 ? launch_tile<kQ4_0, 3>(a, wgs, stream) : launch_tile<kQ4_0, 2>(a, wgs, stream);
    else if (fmt == kQ8_0) e = p.nt == 3 ? launch_tile<kQ8_0, 3>(a, wgs, stream) : launch_tile<kQ8_0, 2>(a, wgs, stream);
#else
    if (fmt == kQ4_0) e = p.nt == 3 ? launch_wave<kQ4_0, 3>(a, wgs, stream) : launch_wave<kQ4_0, 2>(a, wgs, stream);
    else if (fmt == kQ8_0) e = p.nt == 3 ? launch_wave<kQ8_0, 3>(a, wgs, stream) : launch_wave<kQ8_0, 2>(a, wgs, stream);
#endif
    else if (fmt == kI8B64) e = launch_tile<kI8B64, 2>(a, wgs, stream);
    else e = launch_tile<kI8B32, 2>(a, wgs, stream);
    if (e != hipSuccess || p.S == 1) return e;
    return launch_splitk_reduce(static_cast<const float*>(ws), Y[0], size_t(M) * size_t(N[0]), p.S, stream);
}

}  // namespace lq
