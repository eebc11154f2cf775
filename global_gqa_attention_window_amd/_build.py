"""Build the gfx950 shared library libgqa_attn.so in-tree with hipcc (and the
benchmark's calibration kernels, libgqa_calib.so)."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgqa_attn.so")
CALIB = os.path.join(PKG, "libgqa_calib.so")
SOURCES = ["api.hip", "decode.hip", "prefill.hip", "prefill512.hip", "cache_write.hip",
           "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# per-source extras for the prompt and decode-window kernels: their
# matrix-core accumulators stay in ordinary VGPRs (Q sits in AGPRs instead),
# so rescaling them needs no copies between accumulation and arithmetic
# registers; and their step loops must unroll fully (a step index that stays
# dynamic would put the register arrays it indexes into scratch memory),
# beyond clang's default size limit for unroll pragmas
_PROMPT = ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-pragma-unroll-threshold=1000000"]
EXTRA = {"prefill.hip": _PROMPT, "prefill512.hip": _PROMPT, "decode.hip": _PROMPT}
NOISE = "is not a recognized feature for this target"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if NOISE not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    return msgs


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libgqa_attn.so; returns its path."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs, msgs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        msgs += _run([HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src),
                      "-o", obj])
        objs.append(obj)
    tmp = LIB + ".tmp"
    msgs += _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    # the benchmark's calibration kernels, a library of their own
    cobj = os.path.join(objdir, "calib.o")
    msgs += _run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, "calib.hip"), "-o", cobj])
    msgs += _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", cobj, "-o", CALIB + ".tmp"])
    os.replace(CALIB + ".tmp", CALIB)
    if verbose and msgs:
        print("\n".join(msgs))
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
