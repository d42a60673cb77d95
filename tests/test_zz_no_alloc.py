"""lq_gemv_batch_noalloc (the GEMV entry point that allocates nothing: its
split-K workspace is a static array inside the library) against
lq_gemv_batch with a caller workspace, through the C ABI: the same launches,
so the same bits, and both at the oracle's GEMV bar.  Two calls in a row, the
second on a smaller input, so the second finds the first one's leftovers in
the shared array."""
import numpy as np
import pytest
import torch

import gemm_q4_q8_int8_amd as lq
import lqgen
from gemm_q4_q8_int8_amd.device import to_device
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

ORACLE_FMT = {"q4_0": 0, "q8_0": 1, "i8b64": 2, "i8b32": 3}


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    lq.load()
    lq.lq_init()
    yield


def _set(oracle, wl):
    mats = [(m, *m.generate()) for m in wl.mats]
    xs = {k: wl.x(k) for k in wl.xs}
    devs = [(gu.upload(m.fmt, w, s, m.N, m.K), to_device(xs[m.xkey])) for m, w, s in mats]
    return mats, xs, devs


def _run(fn, mats, devs):
    ys = [gu.guarded(m.N) for m, _, _ in mats]
    fn([(gu.FMT[m.fmt], Wd, xd, y, m.N, m.K) for (m, _, _), (Wd, xd), y in zip(mats, devs, ys)])
    torch.cuda.synchronize()
    out = []
    for (m, _, _), y in zip(mats, ys):
        gu.check_guard(y, m.N)
        out.append(y[:m.N].cpu().numpy())
    return out


def test_noalloc_matches_workspace_call(oracle):
    big = lqgen.q8_0_layer_2048(3)                 # 7 matrices, down splits K across workgroups
    small = lqgen.q4_0_ffn_2560x960()              # one smaller matrix, another format
    for name, wl in (("q8_0 decoder layer", big), ("q4_0 2560x960", small)):
        say("noalloc", name)
        mats, xs, devs = _set(oracle, wl)
        got = _run(lq.lq_gemv_batch_noalloc, mats, devs)
        ws = torch.full((lq.lq_gemv_workspace_bytes(),), 0x5A, dtype=torch.uint8, device="cuda")
        want = _run(lambda d: lq.lq_gemv_batch(d, ws=ws), mats, devs)
        for (m, w, s), g, r in zip(mats, got, want):
            assert np.array_equal(g, r), (name, m.name)
            yr, S = oracle.gemv(ORACLE_FMT[m.fmt], w, s, xs[m.xkey], m.N, m.K)
            assert gu.ratio(g, yr, S, gu.GEMV_REL, gu.GEMV_ABS) <= 1.0, (name, m.name)
