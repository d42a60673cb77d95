// liblq C ABI: argument validation, launch configuration and error reporting.
// Every check runs before the first HIP call of an entry point, so a rejected
// call leaves device and stream untouched.
#include "../../include/lq.h"
#include "lq_internal.h"

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <vector>

// Split-K workspace of lq_gemv_batch_noalloc, for callers that cannot
// allocate: part of the library's code object, one copy per device (the GPU
// holds it until the process ends).  Host code never uses this name as an
// address (on the host it is only a stand-in for the symbol): it takes the
// device address from hipGetSymbolAddress, looked up once per device.
static __device__ __align__(256) uint8_t scratch[lq::kGemvWorkspaceBytes];

namespace {

thread_local char g_err[512] = "";

lq_status fail(lq_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

lq_status hip_fail(hipError_t e, const char* what) {
    return fail(LQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool fmt_ok(int32_t f) { return f == LQ_Q4_0 || f == LQ_Q8_0 || f == LQ_I8B64 || f == LQ_I8B32; }
bool has_gguf_form(int32_t f) { return f == LQ_Q4_0 || f == LQ_Q8_0; }
int32_t block_of(int32_t f) { return f == LQ_I8B64 ? 64 : (fmt_ok(f) ? 32 : 0); }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
constexpr int64_t kMaxDim = 2147483647;
// A 64-row tile spans at most 64 * K code bytes; kernels address inside a
// tile with 32-bit offsets.
constexpr int64_t kMaxK = int64_t(1) << 25;

lq_status check_fmt_shape(int32_t fmt, int64_t N, int64_t K) {
    if (!fmt_ok(fmt)) return fail(LQ_ERR_FMT, "unknown weight format %d", fmt);
    if (N < 1 || N > kMaxDim) return fail(LQ_ERR_SHAPE, "N=%lld out of range [1, 2^31-1]", (long long)N);
    if (K < 1 || K > kMaxK) return fail(LQ_ERR_SHAPE, "K=%lld out of range [1, 2^25]", (long long)K);
    if (K % block_of(fmt) != 0)
        return fail(LQ_ERR_SHAPE, "K=%lld is not a multiple of the block size %d", (long long)K, block_of(fmt));
    if (N * (K / 32) > (int64_t(1) << 40)) return fail(LQ_ERR_SHAPE, "matrix too large");
    return LQ_OK;
}

lq_status check_ptr(const void* p, uintptr_t align, const char* name) {
    if (!p) return fail(LQ_ERR_ARG, "%s is NULL", name);
    if (!aligned(p, align)) return fail(LQ_ERR_ALIGN, "%s is not %u-byte aligned", name, unsigned(align));
    return LQ_OK;
}

lq_status check_xdt(int32_t xdt) {
    if (xdt != LQ_F32 && xdt != LQ_F16) return fail(LQ_ERR_DTYPE, "unknown activation dtype %d", xdt);
    return LQ_OK;
}

#define LQ_TRY(expr)                    \
    do {                                \
        const lq_status st__ = (expr);  \
        if (st__ != LQ_OK) return st__; \
    } while (0)

// Per-device compute-unit counts, filled on first use of a device.
std::mutex g_dev_mu;
int g_cus[64] = {0};

lq_status device_cus(int* cus) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(LQ_ERR_HIP, "device index %d unsupported", dev);
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_cus[dev] == 0) {
        int n = 0;
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
        g_cus[dev] = n > 0 ? n : 1;
    }
    *cus = g_cus[dev];
    return LQ_OK;
}

// A GEMV workspace is optional; when given it must hold
// lq_gemv_workspace_bytes() bytes and be 16-byte aligned.
lq_status check_gemv_ws(const void* ws, size_t ws_bytes) {
    if (!ws) return LQ_OK;
    if (ws_bytes < lq::kGemvWorkspaceBytes)
        return fail(LQ_ERR_WORKSPACE, "GEMV workspace of %zu bytes required, %zu given", lq::kGemvWorkspaceBytes,
                    ws_bytes);
    if (!aligned(ws, 16)) return fail(LQ_ERR_ALIGN, "ws is not 16-byte aligned");
    return LQ_OK;
}

// Most tokens lq_matmul sends to the multi-token GEMV; more go to the GEMM.
constexpr int64_t kMatmulGemvMaxTokens = lq::kMultiMaxTokens;

lq_status check_gemv_desc(const lq_gemv_desc& d, int idx) {
    lq_status st = check_fmt_shape(d.fmt, d.N, d.K);
    if (st != LQ_OK) return st;
    st = check_xdt(d.xdt);
    if (st != LQ_OK) return st;
    if (!d.W || !d.x || !d.y) return fail(LQ_ERR_ARG, "descriptor %d: W, x or y is NULL", idx);
    if (!aligned(d.W, 16) || !aligned(d.x, 16))
        return fail(LQ_ERR_ALIGN, "descriptor %d: W and x must be 16-byte aligned", idx);
    if (!aligned(d.y, 4)) return fail(LQ_ERR_ALIGN, "descriptor %d: y must be 4-byte aligned", idx);
    return LQ_OK;
}

// K split of a grouped GEMV launch (single- or multi-token): S[i] workgroups
// share each 64-row tile of matrix i.  When the launch has fewer tiles than
// about LQ_GEMV_WGS_PER_CU workgroups per CU, every matrix is split so that
// its workgroups get about the same number of units (the launch's total work
// spread over that many workgroups), never below min_units per wave (per
// format: gemv_min_units, multi_min_units).  Equal work per workgroup keeps
// a long-K matrix from becoming the tail of the launch.  M[i] tokens of
// partials per row count against the split-K workspace; if they do not fit,
// nothing is split.
void split_k(int min_units, int cus, const std::vector<int64_t>& tiles, const std::vector<int64_t>& nu,
             const std::vector<int64_t>& M, std::vector<int64_t>& S) {
    const size_t n = tiles.size();
    int64_t total_tiles = 0, work = 0;
    for (size_t i = 0; i < n; ++i) {
        total_tiles += tiles[i];
        work += tiles[i] * nu[i];
        S[i] = 1;
    }
    const int64_t target = int64_t(cus) * LQ_GEMV_WGS_PER_CU;
    if (total_tiles >= target) return;
    const double per_wg = double(work) / double(target);   // units per workgroup
    int64_t part = 0, cnt = 0;
    for (size_t i = 0; i < n; ++i) {
        const int64_t cap = std::max<int64_t>(1, nu[i] / (4 * min_units));
        const int64_t want = std::max<int64_t>(1, int64_t(double(nu[i]) / per_wg + 0.5));
        S[i] = std::min(std::min(want, cap), lq::kMaxSlices);
        if (S[i] > 1) {
            part += S[i] * M[i] * tiles[i] * lq::kTileRows;
            cnt += tiles[i];
        }
    }
    if (part > lq::kGemvPartFloats || cnt > lq::kGemvCounters)
        for (size_t i = 0; i < n; ++i) S[i] = 1;
}

// Launch order of a grouped launch's matrices: most K slices per tile first
// (stable).  Workgroups are dispatched, and their loads served by HBM, about
// in launch order, so the split-K round trip of the split matrices (partials,
// arrival counter, ordered sum) overlaps the stream of the others instead of
// trailing the launch.
std::vector<int> split_first(const std::vector<int64_t>& S) {
    std::vector<int> ord(S.size());
    for (size_t i = 0; i < ord.size(); ++i) ord[i] = int(i);
    std::stable_sort(ord.begin(), ord.end(), [&](int p, int q) { return S[p] > S[q]; });
    return ord;
}

// One matrix of a GEMV launch: mt rows of K activations in x (row pitch K),
// mt rows of N outputs in y (row pitch N).
struct GemvJob {
    const void* W;
    const void* x;
    float* y;
    int64_t N;
    int64_t K;
};

// Workspace of a GEMV call: the counters, then the partial sums (NULL when
// the caller gave none: then no launch splits K across workgroups).
struct GemvWs {
    uint64_t* cnt;
    float* part;
};
GemvWs gemv_ws(void* ws) {
    if (!ws) return {nullptr, nullptr};
    uint64_t* c = static_cast<uint64_t*>(ws);
    return {c, reinterpret_cast<float*>(c + lq::kGemvCounters)};
}

// One grouped GEMV launch: up to kMaxBatch matrices of one format and
// activation dtype, each over mt tokens (1 .. gemv_max_tokens with fp16
// activations), K split by split_k when a workspace is given.
lq_status launch_chunk(int fmt, int xdt, int mt, const std::vector<GemvJob>& g, int cus, GemvWs ws,
                       hipStream_t stream) {
    const int n = int(g.size());
    std::vector<int64_t> tiles(n), nu(n), S(n, 1);
    for (int i = 0; i < n; ++i) {
        tiles[i] = (g[i].N + lq::kTileRows - 1) / lq::kTileRows;
        nu[i] = g[i].K / lq::unit_elems(fmt);
    }
    // Few tiles of a multi-part format (even split by rows into
    // unit_parts(fmt) workgroups each, no more workgroups than CUs), short
    // rows: split each tile by rows instead of K (no split-K round trips;
    // see launch_gemv_sub).  Measured on the int8 block-64 decoder layer:
    // q/k/v 5.0 -> 3.8 us, o 4.7 -> 3.6, down 7.0 -> 6.2; gate/up (176 tiles,
    // 704 sub-tile workgroups) was slower, 6.2 -> 7.7, and keeps the K split.
    // The choice does not depend on mt, so each token row of a few-token
    // launch is the one-token result bit for bit.
    int64_t total_tiles = 0, max_nu = 0;
    for (int i = 0; i < n; ++i) {
        total_tiles += tiles[i];
        max_nu = std::max(max_nu, nu[i]);
    }
    if (fmt != LQ_Q4_0 && total_tiles * lq::unit_parts(fmt) <= cus && max_nu <= LQ_GEMV_SUB_MAX_UNITS) {
        const int parts = lq::unit_parts(fmt);
        lq::GemvArgs a = {};
        int64_t wgs = 0;
        for (int i = 0; i < n; ++i) {
            const GemvJob& d = g[i];
            lq::GemvDesc& o = a.d[i];
            o.codes = static_cast<const uint8_t*>(d.W);
            o.scales = static_cast<const uint8_t*>(d.W) + lq::align256(lq::code_plane_bytes(fmt, d.N, d.K));
            o.x = d.x;
            o.y = d.y;
            o.N = int32_t(d.N);
            o.nu = int32_t(nu[i]);
            o.tiles = int32_t(tiles[i]);
            o.S = 1;
            o.wg0 = int32_t(wgs);
            o.tile_bytes = uint32_t(lq::kTileRows * nu[i] * lq::unit_bytes(fmt));
            o.part = nullptr;
            o.cnt = nullptr;
            wgs += tiles[i] * parts;
        }
        lq::fill_wg0_table(a.wg0, a.d, n);
        a.count = n;
        a.total_wgs = int32_t(wgs);
        const hipError_t e = lq::launch_gemv_sub(fmt, xdt, mt, a, stream);
        if (e != hipSuccess) return hip_fail(e, "GEMV launch");
        return LQ_OK;
    }
    split_k(lq::gemv_min_units(fmt), cus, tiles, nu, std::vector<int64_t>(n, mt), S);
    // When every matrix splits K at least LQ_GEMV_WIDE_FROM ways, the launch
    // uses 16-wave workgroups: four of the K slices move inside a workgroup
    // (summed in LDS), leaving fewer or no split-K round trips.
    int waves = 4;
    bool wide = true;
    for (int i = 0; i < n; ++i) wide = wide && S[i] >= LQ_GEMV_WIDE_FROM;
    if (wide) {
        waves = 16;
        for (int i = 0; i < n; ++i) S[i] = (S[i] + 3) / 4;
    }
    // Without a workspace the K slices of a tile stay inside its workgroup.
    if (!ws.cnt)
        for (int i = 0; i < n; ++i) S[i] = 1;
    float* part = ws.part;
    uint64_t* cntp = ws.cnt;
    const std::vector<int> ord = split_first(S);
    lq::GemvArgs a = {};
    int64_t wgs = 0, part_off = 0, cnt_off = 0;
    for (int j = 0; j < n; ++j) {
        const int i = ord[j];
        const GemvJob& d = g[i];
        lq::GemvDesc& o = a.d[j];
        o.codes = static_cast<const uint8_t*>(d.W);
        o.scales = static_cast<const uint8_t*>(d.W) + lq::align256(lq::code_plane_bytes(fmt, d.N, d.K));
        o.x = d.x;
        o.y = d.y;
        o.N = int32_t(d.N);
        o.nu = int32_t(nu[i]);
        o.tiles = int32_t(tiles[i]);
        o.S = int32_t(S[i]);
        o.wg0 = int32_t(wgs);
        o.tile_bytes = uint32_t(lq::kTileRows * nu[i] * lq::unit_bytes(fmt));
        o.part = nullptr;
        o.cnt = nullptr;
        if (S[i] > 1) {
            o.part = part + part_off;
            o.cnt = cntp + cnt_off;
            part_off += S[i] * mt * tiles[i] * lq::kTileRows;
            cnt_off += tiles[i];
        }
        wgs += tiles[i] * S[i];
        if (wgs > INT32_MAX) return fail(LQ_ERR_SHAPE, "too many rows in one grouped launch");
    }
    lq::fill_wg0_table(a.wg0, a.d, n);
    a.tag = lq::next_splitk_tag();
    a.count = n;
    a.total_wgs = int32_t(wgs);
    const hipError_t e = lq::launch_gemv(fmt, xdt, waves, mt, a, stream);
    if (e != hipSuccess) return hip_fail(e, "GEMV launch");
    return LQ_OK;
}

lq_status check_multi_desc(const lq_gemv_multi_desc& d, int idx) {
    lq_status st = check_fmt_shape(d.fmt, d.N, d.K);
    if (st != LQ_OK) return st;
    st = check_xdt(d.xdt);
    if (st != LQ_OK) return st;
    if (d.xdt != LQ_F16)
        return fail(LQ_ERR_UNSUPPORTED, "descriptor %d: multi-token GEMV takes LQ_F16 activations", idx);
    if (d.M < 1 || d.M > lq::kMultiMaxTokens)
        return fail(LQ_ERR_SHAPE, "descriptor %d: M=%lld out of range [1, %d]", idx, (long long)d.M,
                    lq::kMultiMaxTokens);
    if (!d.W || !d.X || !d.Y) return fail(LQ_ERR_ARG, "descriptor %d: W, X or Y is NULL", idx);
    if (!aligned(d.W, 16) || !aligned(d.X, 16))
        return fail(LQ_ERR_ALIGN, "descriptor %d: W and X must be 16-byte aligned", idx);
    if (!aligned(d.Y, 4)) return fail(LQ_ERR_ALIGN, "descriptor %d: Y must be 4-byte aligned", idx);
    return LQ_OK;
}

// One grouped multi-token launch: up to kMaxBatch descriptors of one format.
// The K split follows the single-token rule, with the partials of M tokens
// per row counted against the workspace (no split without one).
lq_status launch_multi_chunk(int fmt, const std::vector<const lq_gemv_multi_desc*>& g, int cus, GemvWs ws,
                             hipStream_t stream) {
    const int n = int(g.size());
    std::vector<int64_t> tiles(n), nu(n), S(n, 1);
    for (int i = 0; i < n; ++i) {
        tiles[i] = (g[i]->N + lq::kTileRows - 1) / lq::kTileRows;
        nu[i] = g[i]->K / lq::unit_elems(fmt);
    }
    std::vector<int64_t> Ms(n);
    for (int i = 0; i < n; ++i) Ms[i] = g[i]->M;
    const int64_t most_tokens = *std::max_element(Ms.begin(), Ms.end());
    split_k(lq::multi_min_units(fmt, most_tokens), cus, tiles, nu, Ms, S);
    if (!ws.cnt)
        for (int i = 0; i < n; ++i) S[i] = 1;
    float* part = ws.part;
    uint64_t* cntp = ws.cnt;
    const std::vector<int> ord = split_first(S);
    lq::MultiArgs a = {};
    int64_t wgs = 0, part_off = 0, cnt_off = 0;
    for (int j = 0; j < n; ++j) {
        const int i = ord[j];
        const lq_gemv_multi_desc& d = *g[i];
        lq::MultiDesc& o = a.d[j];
        o.codes = static_cast<const uint8_t*>(d.W);
        o.scales = static_cast<const uint8_t*>(d.W) + lq::align256(lq::code_plane_bytes(fmt, d.N, d.K));
        o.x = static_cast<const _Float16*>(d.X);
        o.y = d.Y;
        o.N = int32_t(d.N);
        o.K = int32_t(d.K);
        o.nu = int32_t(nu[i]);
        o.tiles = int32_t(tiles[i]);
        o.S = int32_t(S[i]);
        o.M = int32_t(d.M);
        o.vec_y = (aligned(d.Y, 16) && d.N % 4 == 0) ? 1 : 0;
        o.wg0 = int32_t(wgs);
        o.part = nullptr;
        o.cnt = nullptr;
        if (S[i] > 1) {
            o.part = part + part_off;
            o.cnt = cntp + cnt_off;
            part_off += S[i] * d.M * tiles[i] * lq::kTileRows;
            cnt_off += tiles[i];
        }
        wgs += tiles[i] * S[i];
        if (wgs > INT32_MAX) return fail(LQ_ERR_SHAPE, "too many rows in one grouped launch");
    }
    lq::fill_wg0_table(a.wg0, a.d, n);
    a.tag = lq::next_splitk_tag();
    a.count = n;
    a.total_wgs = int32_t(wgs);
    const hipError_t e = lq::launch_gemv_multi(fmt, a, stream);
    return e == hipSuccess ? LQ_OK : hip_fail(e, "multi-token GEMV launch");
}

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {nullptr};

// Device address of this device's `scratch` (looked up on first use).
lq_status scratch_ptr(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(LQ_ERR_HIP, "device index %d unsupported", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(LQ_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return LQ_OK;
}

}  // namespace

namespace lq {
// Tags count up from 1 in the low 48 bits (the counter word keeps 16 bits
// for arrivals): 2^48 launches never wrap in a process's lifetime.
uint64_t next_splitk_tag() {
    static std::atomic<uint64_t> next{1};
    return next.fetch_add(1, std::memory_order_relaxed) & ((uint64_t(1) << 48) - 1);
}
}  // namespace lq

extern "C" {

static_assert(LQ_GEMM_MAX_GROUP == lq::kMaxGemmGroup, "GEMM group size");
static_assert(int(LQ_Q4_0) == int(lq::kQ4_0) && int(LQ_Q8_0) == int(lq::kQ8_0) &&
                  int(LQ_I8B64) == int(lq::kI8B64) && int(LQ_I8B32) == int(lq::kI8B32),
              "format numbering");

int32_t lq_abi_version(void) { return LQ_ABI_VERSION; }

lq_status lq_init(void) {
    int n = 0;
    const hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
    if (n < 1) return fail(LQ_ERR_HIP, "no HIP device present");
    int cus = 0;
    LQ_TRY(device_cus(&cus));
    void* p = nullptr;
    return scratch_ptr(&p);
}

int32_t lq_block_elems(int32_t fmt) { return block_of(fmt); }

size_t lq_packed_bytes(int32_t fmt, int64_t N, int64_t K) {
    if (check_fmt_shape(fmt, N, K) != LQ_OK) return 0;
    return lq::align256(lq::code_plane_bytes(fmt, N, K)) + lq::scale_plane_bytes(fmt, N, K);
}

size_t lq_scale_offset(int32_t fmt, int64_t N, int64_t K) {
    if (check_fmt_shape(fmt, N, K) != LQ_OK) return 0;
    return lq::align256(lq::code_plane_bytes(fmt, N, K));
}

size_t lq_gguf_bytes(int32_t fmt, int64_t N, int64_t K) {
    if (!has_gguf_form(fmt) || check_fmt_shape(fmt, N, K) != LQ_OK) return 0;
    return size_t(N) * size_t(K / 32) * (fmt == LQ_Q4_0 ? 18 : 34);
}

lq_status lq_repack_gguf(int32_t fmt, const void* src, void* dst, int64_t N, int64_t K, void* stream) {
    LQ_TRY(check_fmt_shape(fmt, N, K));
    if (fmt_ok(fmt) && !has_gguf_form(fmt))
        return fail(LQ_ERR_FMT, "fmt=%d (int8 with fp32 scales) has no GGUF form; use lq_pack_planes", fmt);
    LQ_TRY(check_ptr(src, 2, "src"));
    LQ_TRY(check_ptr(dst, 16, "dst"));
    const hipError_t e = lq::launch_repack_gguf(fmt, src, dst, N, K, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LQ_OK : hip_fail(e, "repack launch");
}

lq_status lq_pack_planes(int32_t fmt, const void* codes, const void* scales, void* dst, int64_t N,
                         int64_t K, void* stream) {
    LQ_TRY(check_fmt_shape(fmt, N, K));
    LQ_TRY(check_ptr(codes, 16, "codes"));
    LQ_TRY(check_ptr(scales, 4, "scales"));
    LQ_TRY(check_ptr(dst, 16, "dst"));
    const hipError_t e = lq::launch_pack_planes(fmt, codes, scales, dst, N, K, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LQ_OK : hip_fail(e, "pack launch");
}

lq_status lq_quantize(int32_t fmt, const void* src, int32_t sdt, void* W, int64_t N, int64_t K,
                      void* stream) {
    LQ_TRY(check_fmt_shape(fmt, N, K));
    if (sdt != LQ_F32 && sdt != LQ_F16 && sdt != LQ_BF16)
        return fail(LQ_ERR_DTYPE, "unknown source dtype %d", sdt);
    LQ_TRY(check_ptr(src, 16, "src"));
    LQ_TRY(check_ptr(W, 16, "W"));
    const hipError_t e = lq::launch_quantize(fmt, sdt, src, W, N, K, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LQ_OK : hip_fail(e, "quantize launch");
}

static lq_status dequant_common(int32_t fmt, const void* W, void* out, int64_t N, int64_t K,
                                void* stream, bool f16) {
    LQ_TRY(check_fmt_shape(fmt, N, K));
    LQ_TRY(check_ptr(W, 16, "W"));
    LQ_TRY(check_ptr(out, 16, "out"));
    const hipError_t e = lq::launch_dequant(fmt, f16, W, out, N, K, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LQ_OK : hip_fail(e, "dequant launch");
}

lq_status lq_dequant_f32(int32_t fmt, const void* W, float* out, int64_t N, int64_t K, void* stream) {
    return dequant_common(fmt, W, out, N, K, stream, false);
}

lq_status lq_dequant_f16(int32_t fmt, const void* W, uint16_t* out, int64_t N, int64_t K, void* stream) {
    return dequant_common(fmt, W, out, N, K, stream, true);
}

size_t lq_gemv_workspace_bytes(void) { return lq::kGemvWorkspaceBytes; }

lq_status lq_gemv_batch(const lq_gemv_desc* descs, int32_t count, void* ws, size_t ws_bytes, void* stream) {
    if (!descs) return fail(LQ_ERR_ARG, "descs is NULL");
    if (count < 1) return fail(LQ_ERR_ARG, "count=%d must be >= 1", count);
    for (int32_t i = 0; i < count; ++i) LQ_TRY(check_gemv_desc(descs[i], i));
    LQ_TRY(check_gemv_ws(ws, ws_bytes));
    int cus = 0;
    LQ_TRY(device_cus(&cus));
    const GemvWs w = gemv_ws(ws);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    // Group descriptors that share a kernel (format and activation dtype),
    // keeping their order, and launch each group in chunks of kMaxBatch.
    // Launches on one stream run in order, so they share the workspace.
    std::vector<bool> done(size_t(count), false);
    for (int32_t i = 0; i < count; ++i) {
        if (done[i]) continue;
        std::vector<GemvJob> chunk;
        for (int32_t j = i; j < count; ++j) {
            if (done[j] || descs[j].fmt != descs[i].fmt || descs[j].xdt != descs[i].xdt) continue;
            chunk.push_back({descs[j].W, descs[j].x, descs[j].y, descs[j].N, descs[j].K});
            done[j] = true;
            if (chunk.size() == size_t(lq::kMaxBatch)) {
                LQ_TRY(launch_chunk(descs[i].fmt, descs[i].xdt, 1, chunk, cus, w, st));
                chunk.clear();
            }
        }
        if (!chunk.empty()) LQ_TRY(launch_chunk(descs[i].fmt, descs[i].xdt, 1, chunk, cus, w, st));
    }
    return LQ_OK;
}

lq_status lq_gemv_batch_noalloc(const lq_gemv_desc* descs, int32_t count, void* stream) {
    // Validate everything before the first HIP call, as lq_gemv_batch does;
    // its workspace is this device's `scratch`, which always has the size a
    // GEMV workspace needs (the launch planner splits K only within it).
    if (!descs) return fail(LQ_ERR_ARG, "descs is NULL");
    if (count < 1) return fail(LQ_ERR_ARG, "count=%d must be >= 1", count);
    for (int32_t i = 0; i < count; ++i) LQ_TRY(check_gemv_desc(descs[i], i));
    static_assert(sizeof(scratch) >= lq::kGemvWorkspaceBytes, "scratch holds a GEMV workspace");
    void* p = nullptr;
    LQ_TRY(scratch_ptr(&p));
    return lq_gemv_batch(descs, count, p, sizeof(scratch), stream);
}

lq_status lq_gemv(int32_t fmt, const void* W, const void* x, int32_t xdt, float* y, int64_t N,
                  int64_t K, void* ws, size_t ws_bytes, void* stream) {
    lq_gemv_desc d;
    d.fmt = fmt;
    d.xdt = xdt;
    d.W = W;
    d.x = x;
    d.y = y;
    d.N = N;
    d.K = K;
    return lq_gemv_batch(&d, 1, ws, ws_bytes, stream);
}

lq_status lq_gemv_multi_batch(const lq_gemv_multi_desc* descs, int32_t count, void* ws, size_t ws_bytes,
                              void* stream) {
    if (!descs) return fail(LQ_ERR_ARG, "descs is NULL");
    if (count < 1) return fail(LQ_ERR_ARG, "count=%d must be >= 1", count);
    for (int32_t i = 0; i < count; ++i) LQ_TRY(check_multi_desc(descs[i], i));
    LQ_TRY(check_gemv_ws(ws, ws_bytes));
    int cus = 0;
    LQ_TRY(device_cus(&cus));
    const GemvWs w = gemv_ws(ws);
    // Group by format and kernel, keeping order, in chunks of kMaxBatch.  Up
    // to lq::gemv_max_tokens(fmt) tokens run on the single-token GEMV kernel
    // (a few fp16 dot products per weight on the vector units, still under
    // the weight stream's time), all descriptors of a launch with the same M;
    // more tokens take the matrix-core kernel.
    const auto kernel_of = [](const lq_gemv_multi_desc& d) {
        return d.M <= lq::gemv_max_tokens(d.fmt) ? d.M : int64_t(0);
    };
    std::vector<bool> done(size_t(count), false);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    for (int32_t i = 0; i < count; ++i) {
        if (done[i]) continue;
        const int64_t kern = kernel_of(descs[i]);
        std::vector<const lq_gemv_multi_desc*> chunk;
        std::vector<GemvJob> jobs;
        for (int32_t j = i; j < count; ++j) {
            if (done[j] || descs[j].fmt != descs[i].fmt || kernel_of(descs[j]) != kern) continue;
            done[j] = true;
            if (kern == 0) chunk.push_back(&descs[j]);
            else jobs.push_back({descs[j].W, descs[j].X, descs[j].Y, descs[j].N, descs[j].K});
            if (chunk.size() == size_t(lq::kMaxBatch)) {
                LQ_TRY(launch_multi_chunk(descs[i].fmt, chunk, cus, w, st));
                chunk.clear();
            }
            if (jobs.size() == size_t(lq::kMaxBatch)) {
                LQ_TRY(launch_chunk(descs[i].fmt, LQ_F16, int(kern), jobs, cus, w, st));
                jobs.clear();
            }
        }
        if (!chunk.empty()) LQ_TRY(launch_multi_chunk(descs[i].fmt, chunk, cus, w, st));
        if (!jobs.empty()) LQ_TRY(launch_chunk(descs[i].fmt, LQ_F16, int(kern), jobs, cus, w, st));
    }
    return LQ_OK;
}

lq_status lq_gemv_multi(int32_t fmt, const void* W, const void* X, int32_t xdt, float* Y, int64_t M,
                        int64_t N, int64_t K, void* ws, size_t ws_bytes, void* stream) {
    lq_gemv_multi_desc d;
    d.fmt = fmt;
    d.xdt = xdt;
    d.W = W;
    d.X = X;
    d.Y = Y;
    d.M = M;
    d.N = N;
    d.K = K;
    return lq_gemv_multi_batch(&d, 1, ws, ws_bytes, stream);
}

lq_status lq_quantize_act(const void* X, int32_t xdt, int64_t M, int64_t K, int8_t* q, float* s, int32_t* sum,
                          void* stream) {
    LQ_TRY(check_xdt(xdt));
    if (M < 1 || M > kMaxDim) return fail(LQ_ERR_SHAPE, "M=%lld out of range [1, 2^31-1]", (long long)M);
    if (K < 1 || K > kMaxK || K % 32 != 0)
        return fail(LQ_ERR_SHAPE, "K=%lld must be a multiple of 32 in [32, 2^25]", (long long)K);
    if (M * (K / 32) > (int64_t(1) << 31) - 256) return fail(LQ_ERR_SHAPE, "too many activation blocks");
    LQ_TRY(check_ptr(X, 16, "X"));
    LQ_TRY(check_ptr(q, 16, "q"));
    LQ_TRY(check_ptr(s, 4, "s"));
    LQ_TRY(check_ptr(sum, 4, "sum"));
    const hipError_t e = lq::launch_quantize_act(xdt, X, M, K, q, s, sum, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LQ_OK : hip_fail(e, "activation quantization launch");
}

lq_status lq_gemv_q8act(int32_t fmt, const void* W, const int8_t* q, const float* s, const int32_t* sum, float* Y,
                        int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes, void* stream) {
    LQ_TRY(check_fmt_shape(fmt, N, K));
    if (M < 1 || M > lq::kQ8ActMaxTokens)
        return fail(LQ_ERR_SHAPE, "M=%lld out of range [1, %d]", (long long)M, lq::kQ8ActMaxTokens);
    LQ_TRY(check_ptr(W, 16, "W"));
    LQ_TRY(check_ptr(q, 16, "q"));
    LQ_TRY(check_ptr(s, 4, "s"));
    LQ_TRY(check_ptr(sum, 4, "sum"));
    LQ_TRY(check_ptr(Y, 4, "Y"));
    LQ_TRY(check_gemv_ws(ws, ws_bytes));
    int cus = 0;
    LQ_TRY(device_cus(&cus));
    // q8act_mfma_from(fmt) tokens or more run on the integer matrix cores
    // with the multi-token GEMV's K split; fewer on the vector dot-product
    // kernel with the single-token GEMV's (a split of LQ_GEMV_WIDE_FROM or
    // more ways moves four slices into one 16-wave workgroup, as the GEMV
    // does).  M tokens of partials per row either way.
    const bool mfma = M >= lq::q8act_mfma_from(fmt);
    const int64_t tiles = (N + lq::kTileRows - 1) / lq::kTileRows;
    const int64_t nu = K / lq::unit_elems(fmt);
    std::vector<int64_t> S(1, 1);
    split_k(mfma ? lq::multi_min_units(fmt, M) : lq::gemv_min_units(fmt), cus, {tiles}, {nu}, {M}, S);
    int waves = 4;
    if (!mfma && S[0] >= LQ_GEMV_WIDE_FROM) {
        waves = 16;
        S[0] = (S[0] + 3) / 4;
    }
    const GemvWs w = gemv_ws(ws);
    if (!w.cnt) S[0] = 1;
    if (tiles * S[0] > INT32_MAX) return fail(LQ_ERR_SHAPE, "too many rows");
    lq::Q8ActArgs a = {};
    a.codes = static_cast<const uint8_t*>(W);
    a.scales = static_cast<const uint8_t*>(W) + lq::align256(lq::code_plane_bytes(fmt, N, K));
    a.q = q;
    a.s = s;
    a.sum = sum;
    a.y = Y;
    a.part = S[0] > 1 ? w.part : nullptr;
    a.cnt = S[0] > 1 ? w.cnt : nullptr;
    a.tag = lq::next_splitk_tag();
    a.N = int32_t(N);
    a.nu = int32_t(nu);
    a.tiles = int32_t(tiles);
    a.S = int32_t(S[0]);
    a.M = int32_t(M);
    const hipError_t e = mfma ? lq::launch_gemv_q8act_mfma(fmt, a, static_cast<hipStream_t>(stream))
                              : lq::launch_gemv_q8act(fmt, a, waves, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LQ_OK : hip_fail(e, "activation-quantized GEMV launch");
}

namespace {
size_t gemm_ws(int32_t fmt, int64_t M, int64_t N, int64_t K) { return lq::gemm_workspace_bytes(fmt, M, N, K); }
}  // namespace

size_t lq_gemm_workspace_bytes(int32_t fmt, int64_t M, int64_t N, int64_t K) {
    if (check_fmt_shape(fmt, N, K) != LQ_OK || M < 1 || M > kMaxDim) return 0;
    return gemm_ws(fmt, M, N, K);
}

lq_status lq_gemm(int32_t fmt, const void* W, const void* X, int32_t xdt, float* Y, int64_t M,
                  int64_t N, int64_t K, void* ws, size_t ws_bytes, void* stream) {
    lq_gemm_desc d;
    d.W = W;
    d.Y = Y;
    d.N = N;
    return lq_gemm_batch(fmt, X, xdt, M, K, &d, 1, ws, ws_bytes, stream);
}

lq_status lq_gemm_batch(int32_t fmt, const void* X, int32_t xdt, int64_t M, int64_t K, const lq_gemm_desc* descs,
                        int32_t count, void* ws, size_t ws_bytes, void* stream) {
    if (!descs) return fail(LQ_ERR_ARG, "descs is NULL");
    if (count < 1 || count > LQ_GEMM_MAX_GROUP)
        return fail(LQ_ERR_ARG, "count=%d out of range [1, %d]", count, LQ_GEMM_MAX_GROUP);
    LQ_TRY(check_xdt(xdt));
    if (M < 1 || M > kMaxDim) return fail(LQ_ERR_SHAPE, "M=%lld out of range [1, 2^31-1]", (long long)M);
    if (xdt != LQ_F16) return fail(LQ_ERR_UNSUPPORTED, "lq_gemm takes LQ_F16 activations");
    if (M * K > (int64_t(1) << 40)) return fail(LQ_ERR_SHAPE, "X too large");
    LQ_TRY(check_ptr(X, 16, "X"));
    size_t need = 0;
    for (int i = 0; i < count; ++i) {
        LQ_TRY(check_fmt_shape(fmt, descs[i].N, K));
        LQ_TRY(check_ptr(descs[i].W, 16, "W"));
        LQ_TRY(check_ptr(descs[i].Y, 4, "Y"));
        need = std::max(need, gemm_ws(fmt, M, descs[i].N, K));
    }
    if (count > 1) need = 0;   // one launch, K not split
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(LQ_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need, ws_bytes);
    if (ws && !aligned(ws, 16)) return fail(LQ_ERR_ALIGN, "ws is not 16-byte aligned");
    int cus = 0;
    LQ_TRY(device_cus(&cus));
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const void* W[lq::kMaxGemmGroup];
    float* Y[lq::kMaxGemmGroup];
    int64_t N[lq::kMaxGemmGroup];
    for (int i = 0; i < count; ++i) {
        W[i] = descs[i].W;
        Y[i] = descs[i].Y;
        N[i] = descs[i].N;
    }
    const hipError_t e = lq::launch_gemm_tile(fmt, W, Y, N, count, X, M, K, ws, cus, s);
    return e == hipSuccess ? LQ_OK : hip_fail(e, "GEMM launch");
}

lq_status lq_matmul(int32_t fmt, const void* W, const void* X, int32_t xdt, float* Y, int64_t M,
                    int64_t N, int64_t K, void* ws, size_t ws_bytes, void* stream) {
    // The GEMV paths take ws as their split-K workspace when it is large
    // enough for one, else run without.
    const bool gemv_ws_ok = ws && ws_bytes >= lq::kGemvWorkspaceBytes && aligned(ws, 16);
    void* gws = gemv_ws_ok ? ws : nullptr;
    const size_t gwb = gemv_ws_ok ? ws_bytes : 0;
    if (M == 1) return lq_gemv(fmt, W, X, xdt, Y, N, K, gws, gwb, stream);
    if (M <= kMatmulGemvMaxTokens && xdt == LQ_F16)
        return lq_gemv_multi(fmt, W, X, xdt, Y, M, N, K, gws, gwb, stream);
    return lq_gemm(fmt, W, X, xdt, Y, M, N, K, ws, ws_bytes, stream);
}

const char* lq_status_str(int32_t status) {
    switch (status) {
        case LQ_OK: return "LQ_OK";
        case LQ_ERR_ARG: return "LQ_ERR_ARG";
        case LQ_ERR_SHAPE: return "LQ_ERR_SHAPE";
        case LQ_ERR_ALIGN: return "LQ_ERR_ALIGN";
        case LQ_ERR_FMT: return "LQ_ERR_FMT";
        case LQ_ERR_DTYPE: return "LQ_ERR_DTYPE";
        case LQ_ERR_UNSUPPORTED: return "LQ_ERR_UNSUPPORTED";
        case LQ_ERR_WORKSPACE: return "LQ_ERR_WORKSPACE";
        case LQ_ERR_HIP: return "LQ_ERR_HIP";
        default: return "LQ_ERR_UNKNOWN";
    }
}

const char* lq_last_error(void) { return g_err; }

}  // extern "C"
