// Dequantizing GEMV for decode: y = W x with W in the packed Q4_0 / Q8_0 /
// int8-block-64 layout.
//
// Decode streams every weight once, so the kernel is bound by HBM bandwidth
// ("oxinfer" page, "Performance": decode is memory-bandwidth bound and its
// speed is set by bytes per token).  Design for gfx950:
//   * One launch covers up to 16 matrices (for example every projection of a
//     decoder layer).  Their rows are cut into row iterations of RPI rows per
//     team, each walked in chunks of TP 32-weight units (one step per chunk).
//     A persistent grid (a few workgroups per CU) takes the row iterations
//     grid-stride, so at any moment all workgroups stream neighbouring rows
//     (DRAM-friendly) and every CU stays busy to the end.
//   * All activation vectors of the launch (de-duplicated by the host) are
//     copied into LDS as fp32 once, before the main loop: the loop itself has
//     no barrier and no activation load from global memory.  Each lane copies
//     its unit's 32 values into VGPRs when the matrix or chunk changes.
//   * A team of TP lanes (16, 32 or 64: the smallest that covers a row; long
//     rows are walked in chunks of 64 units) works on one row at a time; lane
//     t of a team owns unit t of the chunk.  Consecutive lanes read
//     consecutive 16-byte code blocks, so each wave load is one contiguous
//     span of the code plane, issued as 128-bit non-temporal loads.
//   * A ring of register buffers keeps the loads of the next steps in flight
//     while the current step computes.
//   * Q4_0 nibbles become exact fp16 values (q - 8) with one v_and_or_b32
//     (nibble into an fp16 mantissa under exponent 2^10) and one v_pk_add_f16
//     per two weights; v_fma_mix_f32 then multiplies that fp16 by the fp32
//     activation into an fp32 accumulator.
//   * int8 codes use sign-extending SDWA byte selects into v_cvt_f32_i32 and an
//     fp32 FMA.
//   * The block scale multiplies the unit's partial sum once (per block, not
//     per weight).  Partial sums of a row are combined across the team with
//     a transposed butterfly: each halving step exchanges half of the rows'
//     partials, so RPI rows cost about RPI + log2(TP) exchanges instead of
//     RPI * log2(TP), and every exchange is a VALU lane permute (DPP or
//     permlane swap), never an LDS round trip.
#include "lq_internal.h"

namespace lq {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// Sum over 32 int8 codes (two 16-byte loads, element order) of c_e * x_e.
__device__ __forceinline__ float dot_i8(const u32x4 c0, const u32x4 c1, const float (&x)[32]) {
    const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
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

// Value held by this lane's exchange partner across lane bit OFF, with VALU
// lane permutes only (no LDS round trip): DPP quad permutes for bits 0 and 1,
// DPP half-row / row mirrors for bits 2 and 3 (lane i <-> 7-i, 15-i: partner
// differs in that bit), and the gfx950 permlane16 / permlane32 swaps for
// bits 4 and 5.  lt is the lane index inside an aligned team (its low bits
// equal the wave lane's).
template <int OFF>
__device__ __forceinline__ float xor_partner(float v, int lt) {
    const uint32_t u = __float_as_uint(v);
    uint32_t r;
    if constexpr (OFF == 1) {
        r = __builtin_amdgcn_update_dpp(0u, u, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    } else if constexpr (OFF == 2) {
        r = __builtin_amdgcn_update_dpp(0u, u, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    } else if constexpr (OFF == 4) {
        r = __builtin_amdgcn_update_dpp(0u, u, 0x141, 0xF, 0xF, false);  // row_half_mirror
    } else if constexpr (OFF == 8) {
        r = __builtin_amdgcn_update_dpp(0u, u, 0x140, 0xF, 0xF, false);  // row_mirror
    } else if constexpr (OFF == 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        r = (lt & 16) ? p[0] : p[1];
    } else {
        static_assert(OFF == 32, "lane exchange offset must be 1..32");
        const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        r = (lt & 32) ? p[0] : p[1];
    }
    return __uint_as_float(r);
}

// One halving step of the transposed butterfly: lanes whose bit OFF is set
// keep the upper half of the N live partials and send the lower half to their
// partner, which does the opposite; each side adds what it receives.
template <int N, int OFF, int RPI>
__device__ __forceinline__ void halve(float (&v)[RPI], int lt) {
    constexpr int H = N / 2;
    const bool upper = (lt & OFF) != 0;
#pragma unroll
    for (int i = 0; i < H; ++i) {
        const float send = upper ? v[i] : v[i + H];
        const float keep = upper ? v[i + H] : v[i];
        v[i] = keep + xor_partner<OFF>(send, lt);
    }
}

template <int N, int OFF, int RPI>
__device__ __forceinline__ void reduce_from(float (&v)[RPI], int lt) {
    if constexpr (OFF >= 1) {
        if constexpr (N > 1) {
            halve<N, OFF, RPI>(v, lt);
            reduce_from<N / 2, OFF / 2, RPI>(v, lt);
        } else {
            v[0] += xor_partner<OFF>(v[0], lt);
            reduce_from<1, OFF / 2, RPI>(v, lt);
        }
    }
}

// Transposed butterfly over the TPW lanes of a team inside one wave: on entry
// every lane holds RPI partials (one per row); on exit the lane whose bits
// (TPW/2, TPW/4, ...) spell r holds the team's total for row r in v[0].
// The partner of a lane differs from it in the bit being reduced, so the
// halving decisions and the final row assignment depend only on the lane's
// own bits, whichever partner permutation is used.
template <int RPI, int TPW>
__device__ __forceinline__ void team_reduce(float (&v)[RPI], int lt) {
    static_assert(RPI == 1 || RPI == 2 || RPI == 4 || RPI == 8, "RPI must be 1, 2, 4 or 8");
    static_assert(TPW >= RPI && TPW <= 64, "a team needs RPI..64 lanes");
    reduce_from<RPI, TPW / 2, RPI>(v, lt);
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

// LDS offset (in floats) of the v-th group of four activations of unit u.
// Lanes of a wave read the same group v of consecutive units; rotating the
// eight groups of a unit by u spreads those reads over all LDS banks instead
// of one 128-byte column.
__device__ __forceinline__ int x_slot(int u, int v) { return u * 32 + ((v + u) & 7) * 4; }

// Position in a launch's work: global row iteration (over all matrices of
// the launch, in order), the matrix it belongs to, its row iteration inside
// that matrix, and the chunk of the row.
struct Pos {
    int gi;
    int di;
    int it;
    int ch;
};

__device__ __forceinline__ Pos pos_of(const GemvBatchArgs& a, int gi) {
    int di = 0;
    while (di + 1 < a.count && gi >= a.d[di + 1].iter0) ++di;
    return Pos{gi, di, gi - a.d[di].iter0, 0};
}

// Next step of this workgroup: the next chunk of the row, else the
// workgroup's next row iteration: grid-stride (all workgroups stream
// neighbouring rows at any moment) or, with LQ_GEMV_CONTIGUOUS, the next row
// iteration of the workgroup's own contiguous range.
#ifndef LQ_GEMV_CONTIGUOUS
#define LQ_GEMV_CONTIGUOUS 0
#endif
__device__ __forceinline__ Pos advance(const GemvBatchArgs& a, const Pos& p, int it_end) {
    if (p.ch + 1 < a.d[p.di].nchunks) return Pos{p.gi, p.di, p.it, p.ch + 1};
    const int gi = p.gi + (LQ_GEMV_CONTIGUOUS ? 1 : int(gridDim.x));
    if (gi >= it_end) return Pos{it_end, a.count, 0, 0};
    if (gi - a.d[p.di].iter0 < a.d[p.di].iters) return Pos{gi, p.di, p.it + (gi - p.gi), 0};
    return pos_of(a, gi);
}

// Scales stay as raw bits until the step is computed: converting them right
// after the load would make the wave wait for the load there (vmcnt is in
// order), stalling on the prefetch it has just issued.
template <int FMT, int RPI>
struct StepBuf {
    static constexpr int CW = FMT == kQ4_0 ? 1 : 2;
    u32x4 code[RPI][CW];
    uint32_t sc[RPI];   // fp32 bits (int8 block-64) or fp16 bits (Q4_0 / Q8_0)
    bool u_ok;          // this lane's unit lies inside the row
};

template <int FMT, int RPI>
__device__ __forceinline__ float scale_of(const StepBuf<FMT, RPI>& b, int r) {
    float s;
    if (FMT == kI8B64) s = __uint_as_float(b.sc[r]);
    else s = (float)__builtin_bit_cast(_Float16, uint16_t(b.sc[r]));
    return b.u_ok ? s : 0.0f;
}

// Loads of one step: ordinary (compiler-visible) loads, so the compiler
// tracks every destination register and places its waits itself.  Addresses
// are a step-uniform base (scalar registers) plus a 32-bit lane offset inside
// the step's rows.
template <int FMT, int TP, int RPI>
__device__ __forceinline__ void load_step(const GemvBatchArgs& a, const Pos& p, int team, int lt,
                                          StepBuf<FMT, RPI>& b) {
    constexpr int TEAMS = kGemvThreads / TP;
    constexpr int CW = StepBuf<FMT, RPI>::CW;
    const GemvDesc& D = a.d[p.di];
    // Lanes past the end of a row or rows past N load a clamped (valid)
    // address and get scale 0; their activations are 0 or their rows are not
    // stored, so nothing they read reaches y.  No divergent branches.
    const int u_raw = p.ch * TP + lt;
    const bool u_ok = u_raw < D.nu;
    const int u = u_ok ? u_raw : D.nu - 1;
    const int row0 = p.it * TEAMS * RPI;
    const int rows_left = D.N - 1 - row0;
    const uint8_t* cbase = D.codes + size_t(row0) * size_t(D.nu) * (16 * CW);
    const uint8_t* sbase = static_cast<const uint8_t*>(D.scales) +
                           size_t(row0) * size_t(FMT == kI8B64 ? (D.nu / 2) * 4 : D.nu * 2);
#pragma unroll
    for (int r = 0; r < RPI; ++r) {
        const int rel_raw = r * TEAMS + team;
        const uint32_t rel = uint32_t(rel_raw <= rows_left ? rel_raw : rows_left);
        const uint32_t unit = rel * uint32_t(D.nu) + uint32_t(u);
        const u32x4* cp = reinterpret_cast<const u32x4*>(cbase + unit * (16u * CW));
#pragma unroll
        for (int c = 0; c < CW; ++c) b.code[r][c] = __builtin_nontemporal_load(cp + c);
        if (FMT == kI8B64)
            b.sc[r] = *reinterpret_cast<const uint32_t*>(
                sbase + (rel * uint32_t(D.nu / 2) + uint32_t(u / 2)) * 4u);
        else
            b.sc[r] = *reinterpret_cast<const uint16_t*>(sbase + unit * 2u);
    }
    b.u_ok = u_ok;
}

// XG selects where activations come from: false = every activation vector of
// the launch staged in LDS before the loop (the host keeps their total within
// kGemvXLdsFloats), true = read from global memory per chunk (rows longer
// than the LDS budget).
template <int FMT, int TP, int RPI, bool XG>
__global__ __launch_bounds__(kGemvThreads) __attribute__((amdgpu_waves_per_eu(LQ_GEMV_WGS_PER_CU))) void gemv_kernel(const GemvBatchArgs args) {
    constexpr int TEAMS = kGemvThreads / TP;
    extern __shared__ float xs[];   // activations of every matrix of the launch (fp32)

    const int tid = threadIdx.x;
    const int team = tid / TP;
    const int lt = tid % TP;
    if (int(blockIdx.x) >= args.total_iters) return;

    if (!XG) {
        // Eight 16-byte loads in flight per thread before their LDS stores, so
        // staging costs a few L2 round trips rather than one per load.
        for (int j = 0; j < args.nx; ++j) {
            const GemvXSrc& X = args.xs[j];
            for (int i0 = tid * 4; i0 < X.K; i0 += kGemvThreads * 4 * 8) {
                f32x4 v[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int i = i0 + q * kGemvThreads * 4;
                    const int ic = i < X.K ? i : X.K - 4;
                    if (X.xdt == kF32) {
                        v[q] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(X.x) + ic);
                    } else {
                        const uint2 h = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(X.x) + ic);
                        const half2_t h0 = as_half2(h.x), h1 = as_half2(h.y);
                        v[q] = f32x4{(float)h0.x, (float)h0.y, (float)h1.x, (float)h1.y};
                    }
                }
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int i = i0 + q * kGemvThreads * 4;
                    if (i < X.K)
                        *reinterpret_cast<f32x4*>(xs + X.lds_off + x_slot(i / 32, (i % 32) / 4)) = v[q];
                }
            }
        }
        __syncthreads();
    }

    float xr[32];
    float acc[RPI];
    int x_di = -1;          // matrix and chunk whose activations are in xr
    int x_ch = -1;

    auto process = [&](const Pos& p, StepBuf<FMT, RPI>& b) {
        const GemvDesc& D = args.d[p.di];
        if (p.di != x_di || p.ch != x_ch) {
            const int u = p.ch * TP + lt;
            if (u >= D.nu) {
#pragma unroll
                for (int e = 0; e < 32; ++e) xr[e] = 0.0f;
            } else if (!XG) {
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    const f32x4 t = *reinterpret_cast<const f32x4*>(xs + D.x_off + x_slot(u, v));
                    xr[4 * v + 0] = t.x;
                    xr[4 * v + 1] = t.y;
                    xr[4 * v + 2] = t.z;
                    xr[4 * v + 3] = t.w;
                }
            } else {
                load_x_unit(D.x, D.xdt, u, true, xr);
            }
            x_di = p.di;
            x_ch = p.ch;
        }
        if (p.ch == 0) {
#pragma unroll
            for (int r = 0; r < RPI; ++r) acc[r] = 0.0f;
        }
#pragma unroll
        for (int r = 0; r < RPI; ++r) {
            float s;
            if (FMT == kQ4_0) s = dot_q4_0(b.code[r][0], xr);
            else s = dot_i8(b.code[r][0], b.code[r][StepBuf<FMT, RPI>::CW - 1], xr);
            acc[r] = __builtin_fmaf(scale_of(b, r), s, acc[r]);
            // Keep each row's unpacking next to its FMAs: interleaving the
            // rows would hold every converted code of the step live at once.
            __builtin_amdgcn_sched_barrier(0);
        }
        if (p.ch == D.nchunks - 1) {
            float v[RPI];
#pragma unroll
            for (int r = 0; r < RPI; ++r) v[r] = acc[r];
            team_reduce<RPI, TP>(v, lt);
            const int rr = reduced_row<RPI, TP>(lt);
            const int row = p.it * TEAMS * RPI + rr * TEAMS + team;
            if ((lt % (TP / RPI)) == 0 && row < D.N) D.y[row] = v[0];
        }
    };

    // A ring of NB register buffers: while one step is computed, the loads of
    // the next NB-1 steps are in flight.  Every computed step is preceded by
    // exactly one issued step (past the end the last step is re-read: cache
    // hits), and the loop body is the same on every trip with its only exit
    // leaving the loop, so the compiler's waits leave the younger steps in
    // flight.
    constexpr int NB = LQ_GEMV_NBUF;
    StepBuf<FMT, RPI> buf[NB];
    Pos q[NB];
    bool qv[NB];
#if LQ_GEMV_CONTIGUOUS
    const int it_begin = int(int64_t(args.total_iters) * blockIdx.x / gridDim.x);
    const int it_end = int(int64_t(args.total_iters) * (blockIdx.x + 1) / gridDim.x);
#else
    const int it_begin = int(blockIdx.x);
    const int it_end = args.total_iters;
#endif
    if (it_begin >= it_end) return;
    Pos issue = pos_of(args, it_begin);
    bool issue_ok = true;
    auto issue_next = [&](int bi) {
        load_step<FMT, TP, RPI>(args, issue, team, lt, buf[bi]);
        q[bi] = issue;
        qv[bi] = issue_ok;
        if (issue_ok) {
            const Pos nx = advance(args, issue, it_end);
            if (nx.gi < it_end) issue = nx;
            else issue_ok = false;
        }
    };
#pragma unroll
    for (int i = 0; i < NB - 1; ++i) issue_next(i);
    while (true) {
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            issue_next((k + NB - 1) % NB);
            if (!qv[k]) goto finished;
            process(q[k], buf[k]);
        }
    }
finished:
    return;
}

template <int FMT, int RPI, bool XG>
hipError_t launch_fmt(const GemvConfig& cfg, const GemvBatchArgs& args, int grid, size_t lds,
                      hipStream_t s) {
    switch (cfg.tp) {
        case 16: hipLaunchKernelGGL((gemv_kernel<FMT, 16, RPI, XG>), dim3(grid), dim3(kGemvThreads), lds, s, args); break;
        case 32: hipLaunchKernelGGL((gemv_kernel<FMT, 32, RPI, XG>), dim3(grid), dim3(kGemvThreads), lds, s, args); break;
        case 64: hipLaunchKernelGGL((gemv_kernel<FMT, 64, RPI, XG>), dim3(grid), dim3(kGemvThreads), lds, s, args); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_x(const GemvConfig& cfg, const GemvBatchArgs& args, int grid, size_t lds,
                    hipStream_t s) {
    if (cfg.x_global) return launch_fmt<FMT, gemv_rpi(FMT), true>(cfg, args, grid, 0, s);
    return launch_fmt<FMT, gemv_rpi(FMT), false>(cfg, args, grid, lds, s);
}

}  // namespace

// Team width: the smallest of 16, 32, 64 lanes that covers a row's units in
// one chunk; rows longer than 64 units are walked in chunks of 64.
// Activations of rows longer than the LDS budget are read from global memory.
GemvConfig gemv_config(int fmt, int nu) {
    GemvConfig c;
    c.tp = nu <= 16 ? 16 : (nu <= 32 ? 32 : 64);
    c.rpi = gemv_rpi(fmt);
    c.rows_per_iter = (kGemvThreads / c.tp) * c.rpi;
    c.x_global = int64_t(nu) * 32 > kGemvXLdsFloats;
    return c;
}

hipError_t launch_gemv(int fmt, const GemvConfig& cfg, const GemvBatchArgs& args, int grid,
                       size_t lds_bytes, hipStream_t stream) {
    switch (fmt) {
        case kQ4_0: return launch_x<kQ4_0>(cfg, args, grid, lds_bytes, stream);
        case kQ8_0: return launch_x<kQ8_0>(cfg, args, grid, lds_bytes, stream);
        case kI8B64: return launch_x<kI8B64>(cfg, args, grid, lds_bytes, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lq
