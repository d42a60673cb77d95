"""Build liblq.so (the HIP library) in-tree with hipcc for gfx950.

    python -m gemm_q4_q8_int8_amd.build        # or build() from Python

Every HIP source is compiled with packed-fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops): ordinary float code is
then never turned into v_pk_*_f32.  No fast-math flags: the kernels rely on
IEEE fp32 / fp16 arithmetic with denormals kept.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblq.so")
SOURCES = ["lq_api.hip", "lq_gemv.hip", "lq_multi.hip", "lq_q8act.hip", "lq_convert.hip", "lq_gemm.hip"]
ARCH = os.environ.get("LQ_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Werror", "-Wno-unused-command-line-argument"]


# Per-source extra flags.  The multi-token GEMVs (fp16 and integer) take
# their MFMA results in ordinary VGPRs (the compiler otherwise routes them
# through accumulation registers and copies each one back).
EXTRA = {"lq_multi.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "lq_q8act.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass reports the packed-fp32 target feature as unknown; that
    # line is expected and harmless.
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if err:
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
