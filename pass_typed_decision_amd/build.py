"""Builds libblink.so in-tree: the host packer and the gfx950 HIP kernels, one shared library.

Run as ``python -m pass_typed_decision_amd.build``. Every HIP translation unit is compiled for
gfx950 only, with packed FP32 instructions disabled.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libblink.so")
SOURCES = ["blink_host.cpp", "blink_attention.hip", "blink_attention_plain.hip",
           "blink_readout.hip", "blink_scoring.hip"]
# Per-source flags on top of HIP_FLAGS. The attention kernel's main build uses the ILP-first
# instruction scheduler, which measured 1-2% faster on the matrix-bound launches (bitwise the
# same results); its second build (blink_attention_plain.hip) keeps the default scheduler,
# 3-4% faster on prefix-free requests of short tails.
SOURCE_FLAGS = {"blink_attention.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}
ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # The kernels' bodies are compiled in the device pass only, so the host pass sees their
    # helpers unused.
    "-Wno-unused-function",
    "-Wno-unneeded-internal-declaration",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Matrix-core results in VGPRs: the attention softmax reads its score accumulators with
    # ordinary vector instructions, and the Q fragments it pins in AGPRs feed MFMAs directly.
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _run(cmd, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compiles every source (each with its own flags) and links libblink.so next to this
    file; returns its path."""
    import tempfile

    tmp = LIB + f".tmp{os.getpid()}"
    with tempfile.TemporaryDirectory(prefix="blink_build_") as objdir:
        objs = []
        for src in SOURCES:
            obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
            _run([hipcc(), *HIP_FLAGS, *SOURCE_FLAGS.get(src, []), *extra_flags, "-x", "hip",
                  "-c", "-o", obj, os.path.join(CSRC, src)], verbose)
            objs.append(obj)
        try:
            _run([hipcc(), f"--offload-arch={ARCH}", "-fPIC", "-shared", "-o", tmp, *objs],
                 verbose)
        except RuntimeError:
            if os.path.exists(tmp):
                os.remove(tmp)
            raise
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
