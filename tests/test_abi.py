"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, reports layout sizes, and rejects bad arguments with the
documented status before touching HIP."""
import os
import re

import pytest

import gemm_q4_q8_int8_amd as lq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lq.h")

OK, ARG, SHAPE, ALIGN, FMT, DTYPE, UNSUP, WS, HIP = range(9)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(lq.LIB_PATH):
        from gemm_q4_q8_int8_amd import build
        build.build()
    return lq.load()


def test_exports_every_declared_symbol(L):
    text = open(HEADER).read()
    declared = sorted(set(re.findall(r"\b(lq_[a-z0-9_]+)\s*\(", text)))
    assert declared, "no declarations parsed"
    assert sorted(lq.EXPORTS) == declared
    for name in declared:
        assert hasattr(L, name), name


def test_version_and_names(L):
    assert lq.lq_abi_version() == 8
    names = [lq.lq_status_str(s) for s in range(9)]
    assert names == ["LQ_OK", "LQ_ERR_ARG", "LQ_ERR_SHAPE", "LQ_ERR_ALIGN", "LQ_ERR_FMT",
                     "LQ_ERR_DTYPE", "LQ_ERR_UNSUPPORTED", "LQ_ERR_WORKSPACE", "LQ_ERR_HIP"]


def _align256(v):
    return (v + 255) // 256 * 256


def test_layout_sizes(L):
    for N, K in ((2560, 960), (151936, 896), (1, 32), (3, 96)):
        nb = K // 32
        assert lq.lq_scale_offset(lq.LQ_Q4_0, N, K) == _align256(16 * N * nb)
        assert lq.lq_packed_bytes(lq.LQ_Q4_0, N, K) == _align256(16 * N * nb) + 2 * N * nb
        assert lq.lq_packed_bytes(lq.LQ_Q8_0, N, K) == _align256(32 * N * nb) + 2 * N * nb
        assert lq.lq_gguf_bytes(lq.LQ_Q4_0, N, K) == 18 * N * nb
        assert lq.lq_gguf_bytes(lq.LQ_Q8_0, N, K) == 34 * N * nb
    assert lq.lq_packed_bytes(lq.LQ_I8B64, 5632, 2048) == _align256(5632 * 2048) + 4 * 5632 * 32
    assert lq.lq_gguf_bytes(lq.LQ_I8B64, 64, 64) == 0
    assert lq.lq_packed_bytes(lq.LQ_I8B64, 4, 96) == 0          # K not a multiple of 64
    # the "oxinfer" page's Q8: 36 bytes per 32 weights (int8 codes + fp32 scale)
    assert lq.lq_packed_bytes(lq.LQ_I8B32, 4096, 4096) == _align256(4096 * 4096) + 4096 * 4096 * 36 // 32 - 4096 * 4096
    assert lq.lq_gguf_bytes(lq.LQ_I8B32, 64, 64) == 0
    assert lq.lq_block_elems(lq.LQ_I8B32) == 32 and lq.lq_block_elems(4) == 0
    assert lq.lq_packed_bytes(7, 4, 64) == 0
    assert lq.lq_packed_bytes(lq.LQ_Q4_0, 0, 64) == 0
    assert [lq.lq_block_elems(f) for f in (0, 1, 2, 3, 4)] == [32, 32, 64, 32, 0]
    # the packed bytes of a workload equal its GGUF bytes plus alignment padding
    assert lq.lq_packed_bytes(lq.LQ_Q4_0, 151936, 896) - lq.lq_gguf_bytes(lq.LQ_Q4_0, 151936, 896) < 256


A16 = 0x100000     # a 16-byte aligned address that is never dereferenced: every
                   # call below carries at least one invalid argument


def test_rejections_before_any_hip_call(L):
    g = L
    assert g.lq_gemv(9, A16, A16, 0, A16, 4, 32, None, 0, None) == FMT
    assert g.lq_gemv(0, A16, A16, 0, A16, 0, 32, None, 0, None) == SHAPE
    assert g.lq_gemv(0, A16, A16, 0, A16, -3, 32, None, 0, None) == SHAPE
    assert g.lq_gemv(0, A16, A16, 0, A16, 4, 48, None, 0, None) == SHAPE
    assert g.lq_gemv(2, A16, A16, 0, A16, 4, 96, None, 0, None) == SHAPE       # int8 block 64
    assert g.lq_gemv(0, A16, A16, 0, A16, 4, 2**25 + 32, None, 0, None) == SHAPE   # K above 2^25
    assert g.lq_gemv(0, A16, A16, 0, A16, 2 ** 31, 32, None, 0, None) == SHAPE
    assert g.lq_gemv(0, None, A16, 0, A16, 4, 32, None, 0, None) == ARG
    assert g.lq_gemv(0, A16 + 8, A16, 0, A16, 4, 32, None, 0, None) == ALIGN
    assert g.lq_gemv(0, A16, A16 + 4, 0, A16, 4, 32, None, 0, None) == ALIGN
    assert g.lq_gemv(0, A16, A16, 0, A16 + 2, 4, 32, None, 0, None) == ALIGN
    assert g.lq_gemv(0, A16, A16, 5, A16, 4, 32, None, 0, None) == DTYPE
    assert "dtype" in lq.lq_last_error()
    # batch: count and per-descriptor validation
    d = (lq.lq_gemv_desc * 2)()
    d[0] = lq.lq_gemv_desc(0, 0, A16, A16, A16, 4, 32)
    d[1] = lq.lq_gemv_desc(0, 0, A16, A16, A16, 4, 40)
    assert g.lq_gemv_batch(d, 0, None, 0, None) == ARG
    assert g.lq_gemv_batch(None, 1, None, 0, None) == ARG
    assert g.lq_gemv_batch(d, 2, None, 0, None) == SHAPE
    # GEMV workspace: optional, but when given at least lq_gemv_workspace_bytes(), 16-byte aligned
    wsb = lq.lq_gemv_workspace_bytes()
    assert wsb == (1 << 16) * 8 + (1 << 20) * 4
    d[1] = lq.lq_gemv_desc(0, 0, A16, A16, A16, 4, 64)
    assert g.lq_gemv_batch(d, 2, A16, wsb - 1, None) == WS
    assert g.lq_gemv_batch(d, 2, A16 + 8, wsb, None) == ALIGN
    assert g.lq_gemv(0, A16, A16, 0, A16, 4, 32, A16, 64, None) == WS
    assert g.lq_gemv_multi(0, A16, A16, 1, A16, 4, 64, 32, A16, 16, None) == WS
    assert g.lq_gemv_batch_noalloc(None, 1, None) == ARG
    assert g.lq_gemv_batch_noalloc(d, 0, None) == ARG
    d[1] = lq.lq_gemv_desc(0, 0, A16, A16, A16, 4, 40)
    assert g.lq_gemv_batch_noalloc(d, 2, None) == SHAPE
    # gemm
    assert g.lq_gemm(0, A16, A16, 0, A16, 16, 32, 32, None, 0, None) == UNSUP     # fp32 X
    assert g.lq_gemm(2, A16, A16, 1, A16, 16, 32, 32, None, 0, None) == SHAPE     # int8 block 64
    assert g.lq_gemm(1, A16, A16, 1, A16 + 2, 16, 32, 32, None, 0, None) == ALIGN
    assert g.lq_gemm(0, A16, A16, 1, A16, 0, 32, 32, None, 0, None) == SHAPE
    assert g.lq_gemm(0, A16, A16 + 2, 1, A16, 16, 32, 32, None, 0, None) == ALIGN
    assert g.lq_gemm(0, A16, A16, 7, A16, 16, 32, 32, None, 0, None) == DTYPE
    assert g.lq_matmul(0, A16, A16, 1, A16, 0, 32, 32, None, 0, None) == SHAPE
    # grouped gemm: count, descriptor and per-matrix validation
    gd = (lq.lq_gemm_desc * 5)()
    for i in range(5):
        gd[i] = lq.lq_gemm_desc(A16, A16, 64)
    assert g.lq_gemm_batch(0, A16, 1, 16, 64, None, 1, None, 0, None) == ARG
    assert g.lq_gemm_batch(0, A16, 1, 16, 64, gd, 0, None, 0, None) == ARG
    assert g.lq_gemm_batch(0, A16, 1, 16, 64, gd, lq.LQ_GEMM_MAX_GROUP + 1, None, 0, None) == ARG
    assert g.lq_gemm_batch(0, A16, 0, 16, 64, gd, 2, None, 0, None) == UNSUP     # fp32 X
    assert g.lq_gemm_batch(0, A16 + 2, 1, 16, 64, gd, 2, None, 0, None) == ALIGN
    gd[1] = lq.lq_gemm_desc(A16, A16, 0)
    assert g.lq_gemm_batch(0, A16, 1, 16, 64, gd, 2, None, 0, None) == SHAPE
    gd[1] = lq.lq_gemm_desc(A16 + 4, A16, 64)
    assert g.lq_gemm_batch(0, A16, 1, 16, 64, gd, 2, None, 0, None) == ALIGN
    gd[1] = lq.lq_gemm_desc(A16, None, 64)
    assert g.lq_gemm_batch(0, A16, 1, 16, 64, gd, 2, None, 0, None) == ARG
    # multi-token GEMV: fp16 activations, 1 <= M <= 16
    assert g.lq_gemv_multi(0, A16, A16, 0, A16, 4, 64, 32, None, 0, None) == UNSUP
    assert g.lq_gemv_multi(0, A16, A16, 1, A16, 0, 64, 32, None, 0, None) == SHAPE
    assert g.lq_gemv_multi(0, A16, A16, 1, A16, 17, 64, 32, None, 0, None) == SHAPE
    assert g.lq_gemv_multi(2, A16, A16, 1, A16, 4, 64, 32, None, 0, None) == SHAPE   # int8 block 64
    assert g.lq_gemv_multi(9, A16, A16, 1, A16, 4, 64, 32, None, 0, None) == FMT
    assert g.lq_gemv_multi(0, A16, A16 + 8, 1, A16, 4, 64, 32, None, 0, None) == ALIGN
    assert g.lq_gemv_multi(0, A16, A16, 1, A16 + 1, 4, 64, 32, None, 0, None) == ALIGN
    assert g.lq_gemv_multi(0, A16, None, 1, A16, 4, 64, 32, None, 0, None) == ARG
    assert g.lq_gemv_multi(0, A16, A16, 3, A16, 4, 64, 32, None, 0, None) == DTYPE
    assert g.lq_matmul(0, A16, A16, 1, A16, 4, 64, 48, None, 0, None) == SHAPE
    md = (lq.lq_gemv_multi_desc * 2)()
    md[0] = lq.lq_gemv_multi_desc(0, 1, A16, A16, A16, 4, 64, 32)
    md[1] = lq.lq_gemv_multi_desc(1, 1, A16, A16, A16, 17, 64, 32)
    assert g.lq_gemv_multi_batch(md, 0, None, 0, None) == ARG
    assert g.lq_gemv_multi_batch(None, 1, None, 0, None) == ARG
    assert g.lq_gemv_multi_batch(md, 2, None, 0, None) == SHAPE          # second descriptor: M = 17
    md[1] = lq.lq_gemv_multi_desc(1, 0, A16, A16, A16, 4, 64, 32)
    assert g.lq_gemv_multi_batch(md, 2, None, 0, None) == UNSUP          # fp32 activations
    assert "descriptor 1" in lq.lq_last_error()
    # activation quantization: K a multiple of 32, q 16-byte aligned, s / sum 4-byte
    assert g.lq_quantize_act(A16, 2, 2, 64, A16, A16, A16, None) == DTYPE
    assert g.lq_quantize_act(A16, 0, 0, 64, A16, A16, A16, None) == SHAPE
    assert g.lq_quantize_act(A16, 0, 2, 48, A16, A16, A16, None) == SHAPE
    assert g.lq_quantize_act(A16, 0, 2, 2 ** 25 + 32, A16, A16, A16, None) == SHAPE
    assert g.lq_quantize_act(A16, 0, 2 ** 22, 2 ** 14, A16, A16, A16, None) == SHAPE   # 2^31 blocks
    assert g.lq_quantize_act(A16 + 4, 0, 2, 64, A16, A16, A16, None) == ALIGN
    assert g.lq_quantize_act(A16, 0, 2, 64, A16 + 4, A16, A16, None) == ALIGN
    assert g.lq_quantize_act(A16, 0, 2, 64, A16, A16 + 2, A16, None) == ALIGN
    assert g.lq_quantize_act(A16, 0, 2, 64, A16, A16, None, None) == ARG
    # activation-quantized GEMV: 1 <= M <= 16, K a multiple of the weight block
    assert g.lq_gemv_q8act(9, A16, A16, A16, A16, A16, 2, 64, 64, None, 0, None) == FMT
    assert g.lq_gemv_q8act(0, A16, A16, A16, A16, A16, 0, 64, 64, None, 0, None) == SHAPE
    assert g.lq_gemv_q8act(0, A16, A16, A16, A16, A16, 17, 64, 64, None, 0, None) == SHAPE
    assert g.lq_gemv_q8act(2, A16, A16, A16, A16, A16, 2, 64, 96, None, 0, None) == SHAPE   # int8 block 64
    assert g.lq_gemv_q8act(0, A16 + 8, A16, A16, A16, A16, 2, 64, 64, None, 0, None) == ALIGN
    assert g.lq_gemv_q8act(0, A16, A16 + 8, A16, A16, A16, 2, 64, 64, None, 0, None) == ALIGN
    assert g.lq_gemv_q8act(0, A16, A16, A16 + 1, A16, A16, 2, 64, 64, None, 0, None) == ALIGN
    assert g.lq_gemv_q8act(0, A16, A16, A16, None, A16, 2, 64, 64, None, 0, None) == ARG
    assert g.lq_gemv_q8act(0, A16, A16, A16, A16, A16 + 2, 2, 64, 64, None, 0, None) == ALIGN
    assert g.lq_gemv_q8act(0, A16, A16, A16, A16, A16, 2, 64, 64, A16, 64, None) == WS
    # load-time quantization
    assert g.lq_quantize(9, A16, 0, A16, 4, 64, None) == FMT
    assert g.lq_quantize(0, A16, 3, A16, 4, 64, None) == DTYPE
    assert g.lq_quantize(2, A16, 2, A16, 4, 96, None) == SHAPE
    assert g.lq_quantize(1, A16 + 2, 1, A16, 4, 64, None) == ALIGN
    assert g.lq_quantize(1, A16, 1, None, 4, 64, None) == ARG
    # conversions
    assert g.lq_repack_gguf(2, A16, A16, 4, 64, None) == FMT
    assert g.lq_repack_gguf(0, A16 + 1, A16, 4, 64, None) == ALIGN
    assert g.lq_repack_gguf(0, A16, A16 + 8, 4, 64, None) == ALIGN
    assert g.lq_pack_planes(2, A16, None, A16, 4, 64, None) == ARG
    assert g.lq_dequant_f32(0, A16, A16 + 4, 4, 64, None) == ALIGN
    assert g.lq_dequant_f16(1, A16, A16, 4, 33, None) == SHAPE


def test_gemm_accepts_activations_above_4gib(L):
    """X of M K 2 >= 2^32 bytes is a valid GEMM (byte offsets into X are
    64-bit): on a machine without a GPU the call gets past every argument
    check and fails only at the first HIP call."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: the call would run (the GPU tests cover it)")
    M, N, K = (1 << 20) + 37, 64, 2048
    assert lq.lq_gemm_workspace_bytes(lq.LQ_Q4_0, M, N, K) == 0
    assert L.lq_gemm(0, A16, A16, 1, A16, M, N, K, None, 0, None) == HIP
    assert L.lq_gemm(0, A16, A16, 1, A16, 1 << 22, 64, 1 << 13, None, 0, None) == HIP   # 64 GiB of X


def test_init_without_device_reports_hip_error(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert L.lq_init() == HIP
    assert lq.lq_last_error() != ""


def test_binding_fails_loudly_without_library(tmp_path):
    old = lq._lib
    try:
        lq._lib = None
        with pytest.raises(lq.LibraryNotBuilt):
            lq.load(str(tmp_path / "missing.so"))
    finally:
        lq._lib = old
