// Prefill GEMM for Q4_0 weights: Y[M x N] = X[M x K] * W[N x K]^T.
//
// Prefill is compute-bound ("oxinfer" page, "Performance"), and the GPU
// kernels the page describes dequantize the weight tile into on-chip memory
// before the dense contraction ("Platforms and accelerators": 64x64 tile per
// threadgroup, weights dequantized to f32 in threadgroup memory).  On gfx950
// the dense step is the fp16 matrix core instruction v_mfma_f32_32x32x16_f16
// (fp32 accumulate), so the tile is dequantized to fp16 instead of fp32:
//   * each workgroup owns a 128 x 128 output tile and walks K in steps of 64
//     (two Q4_0 blocks per weight row);
//   * one thread turns one Q4_0 block (16 code bytes + fp16 scale) into 32
//     fp16 weights RN_fp16((q - 8) * d): v_perm_b32 places each nibble under
//     the fp16 exponent 2^10, v_pk_add_f16 removes 1032 (exact q - 8) and
//     v_pk_mul_f16 applies d with one rounding;
//   * X rows are copied into LDS as fp16; the next step's global loads are
//     issued before the current step's matrix instructions;
//   * four waves each own a 64 x 64 sub-tile (2 x 2 MFMA tiles of 32 x 32).
#include "lq_internal.h"

namespace lq {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int LDK = BK + 8;     // LDS row pitch in halves (pads rows off the same banks)
constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t bits(half2_t h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ half2_t as_half2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// 32 fp16 weights of one Q4_0 block in element order, two per dword.
__device__ __forceinline__ void dequant_q4_0_f16(const u32x4 c, const half2_t dd, uint32_t (&out)[16]) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    const half2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
    const uint32_t kExp = 0x64646464u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = w[i] & 0x0F0F0F0Fu;          // q of elements 4i .. 4i+3
        const uint32_t hi = (w[i] >> 4) & 0x0F0F0F0Fu;   // q of elements 16+4i .. 16+4i+3
        // v_perm_b32 byte selectors: 0-3 pick bytes of `lo`/`hi`, 4 picks 0x64.
        out[2 * i + 0] = bits((as_half2(__builtin_amdgcn_perm(kExp, lo, 0x04010400u)) - off) * dd);
        out[2 * i + 1] = bits((as_half2(__builtin_amdgcn_perm(kExp, lo, 0x04030402u)) - off) * dd);
        out[8 + 2 * i + 0] = bits((as_half2(__builtin_amdgcn_perm(kExp, hi, 0x04010400u)) - off) * dd);
        out[8 + 2 * i + 1] = bits((as_half2(__builtin_amdgcn_perm(kExp, hi, 0x04030402u)) - off) * dd);
    }
}

__global__ __launch_bounds__(kThreads) void gemm_q4_0_kernel(const uint8_t* __restrict__ W,
                                                            size_t scale_off,
                                                            const _Float16* __restrict__ X,
                                                            float* __restrict__ Y,
                                                            int M, int N, int K) {
    __shared__ __attribute__((aligned(16))) _Float16 As[BM][LDK];
    __shared__ __attribute__((aligned(16))) _Float16 Bs[BN][LDK];

    const int tid = threadIdx.x;
    const int wave = tid / 64;
    const int lane = tid % 64;
    const int n0 = blockIdx.x * BN;
    const int m0 = blockIdx.y * BM;
    const int wm = wave / 2;
    const int wn = wave % 2;
    const int nb = K / 32;

    const _Float16* scales = reinterpret_cast<const _Float16*>(W + scale_off);

    // X loader: row tid/2, 32 halves starting at (tid%2)*32 of the K step.
    const int xr = tid / 2;
    const int xc = (tid % 2) * 32;
    const bool x_ok = m0 + xr < M;
    const _Float16* xrow = X + size_t(x_ok ? m0 + xr : 0) * size_t(K) + xc;
    // W loader: row tid/2, block tid%2 of the K step.
    const int wr = tid / 2;
    const int wb = tid % 2;
    const bool w_ok = n0 + wr < N;
    // Tiled layout: unit u of this row sits at code0 + u * ustride bytes and
    // its scale at scale0 + u * (ustride / 16).
    const TiledPos wpos = tiled_pos(kQ4_0, N, nb, w_ok ? n0 + wr : 0, wb);
    const uint8_t* wcode = W + wpos.code;
    const _Float16* wscale = scales + wpos.scale;
    const uint32_t ustride = wpos.part_stride;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    u32x4 xv[4];
    u32x4 cv;
    _Float16 d;
    auto load_step = [&](int k0) {
        if (x_ok && k0 + xc < K) {
            const u32x4* p = reinterpret_cast<const u32x4*>(xrow + k0);
#pragma unroll
            for (int v = 0; v < 4; ++v) xv[v] = p[v];
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v) xv[v] = u32x4{0u, 0u, 0u, 0u};
        }
        if (w_ok && k0 + wb * 32 < K) {   // K is a multiple of 32, not always of 64
            const uint32_t ku = uint32_t(k0 / 32);
            cv = *reinterpret_cast<const u32x4*>(wcode + size_t(ku) * ustride);
            d = wscale[size_t(ku) * (ustride / 16)];
        } else {
            cv = u32x4{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
            d = (_Float16)0.0f;
        }
    };

    load_step(0);
    for (int k0 = 0; k0 < K; k0 += BK) {
        uint32_t wv[16];
        const half2_t dd = {d, d};
        dequant_q4_0_f16(cv, dd, wv);
        __syncthreads();  // previous step's reads of As/Bs are done
        {
            u32x4* ap = reinterpret_cast<u32x4*>(&As[xr][xc]);
#pragma unroll
            for (int v = 0; v < 4; ++v) ap[v] = xv[v];
            u32x4* bp = reinterpret_cast<u32x4*>(&Bs[wr][wb * 32]);
#pragma unroll
            for (int v = 0; v < 4; ++v) bp[v] = u32x4{wv[4 * v], wv[4 * v + 1], wv[4 * v + 2], wv[4 * v + 3]};
        }
        __syncthreads();
        if (k0 + BK < K) load_step(k0 + BK);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            half8_t a[2], b[2];
            const int kk = ks * 16 + (lane / 32) * 8;
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = *reinterpret_cast<const half8_t*>(&As[wm * 64 + i * 32 + lane % 32][kk]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[j] = *reinterpret_cast<const half8_t*>(&Bs[wn * 64 + j * 32 + lane % 32][kk]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }

    // 32x32 accumulator layout: register r of lane l is row 8*(r/4) + 4*(l/32) + r%4,
    // column l%32.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 64 + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
                const int n = n0 + wn * 64 + j * 32 + lane % 32;
                if (m < M && n < N) Y[size_t(m) * size_t(N) + n] = acc[i][j][r];
            }
}

}  // namespace

size_t gemm_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_gemm_q4_0(const void* W, const void* X, float* Y, int64_t M, int64_t N,
                            int64_t K, void*, size_t, int, hipStream_t stream) {
    const size_t off = align256(code_plane_bytes(kQ4_0, N, K));
    const dim3 grid(unsigned((N + BN - 1) / BN), unsigned((M + BM - 1) / BM));
    hipLaunchKernelGGL(gemm_q4_0_kernel, grid, dim3(kThreads), 0, stream,
                       static_cast<const uint8_t*>(W), off, static_cast<const _Float16*>(X), Y,
                       int(M), int(N), int(K));
    return hipGetLastError();
}

}  // namespace lq
