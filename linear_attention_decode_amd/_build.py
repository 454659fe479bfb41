"""Build libreplayssm.so (the HIP kernels and their C ABI) for gfx950 with hipcc.

Every .hip file under csrc/ is compiled to an object in parallel and linked
into one shared library next to this file.  Packed-fp32 instruction
selection is turned off for device code (-packed-fp32-ops)."""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libreplayssm.so")
BUILD = os.path.join(HERE, "_build")
ARCH = "gfx950"

CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(HERE, "..", "include")]


# Per-file extra flags.  step.hip, step_copy.hip, verify_step.hip, flush.hip, flush_shared.hip,
# gdn.hip: one lane per wavefront or workgroup adds to an arrival counter and needs the old value
# only at its very end; the atomic optimizer would rewrite that add into a wave-wide form whose
# readfirstlane waits for the atomic (and every load before it) where it is issued.
EXTRA = {f: ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]
         for f in ("step.hip", "step_copy.hip", "verify_step.hip", "flush.hip", "flush_shared.hip", "gdn.hip")}
# flush_shared.hip: MFMA accumulators in VGPRs (the AGPR form copied every
# element in and out of the accumulators).
EXTRA["flush_shared.hip"] += ["-mllvm", "-amdgpu-mfma-vgpr-form"]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]

    def compile_one(pair):
        src, obj = pair
        cmd = [_hipcc(), *CFLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(compile_one, zip(srcs, objs)))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
