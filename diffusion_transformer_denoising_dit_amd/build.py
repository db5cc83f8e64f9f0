"""Build ``libdit.so`` (gfx950) in-tree with hipcc.

Every ``csrc/*.hip`` file is compiled to an object under ``_build/`` (in
parallel), then linked into ``diffusion_transformer_denoising_dit_amd/libdit.so``.
Packed-fp32 instructions are disabled on the device pass
(``-target-feature -packed-fp32-ops``); the host pass warns that it does not
know the feature, which is harmless.

    python -m diffusion_transformer_denoising_dit_amd.build
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdit.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-file device flags.  attention.hip keeps its MFMA accumulators in VGPRs
# (its softmax phase reads the scores with VALU instructions, and the AGPR form
# would copy every accumulator register across the register files each tile)
# and is built without NaN semantics (its scores are never NaN), which lets
# the compiler fuse its maxima into v_max3_f32 without quieting operations.
FILE_FLAGS = {
    "attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"],
}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdit.so)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source and link libdit.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))

    def compile_one(pair):
        src, obj = pair
        return _run([hipcc, *COMMON_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src,
                     "-o", obj])

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        logs = list(ex.map(compile_one, zip(srcs, objs)))
    tmp = LIB + ".tmp"
    logs.append(_run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]))
    os.replace(tmp, LIB)
    if verbose:
        for l in logs:
            if l.strip():
                print(l)
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
