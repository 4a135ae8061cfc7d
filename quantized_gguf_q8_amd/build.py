"""Build libggq.so for gfx950 with hipcc (in-tree, no JIT cache).

Every .hip file under csrc/ is compiled to an object in parallel and linked into
quantized_gguf_q8_amd/libggq.so.  Packed-fp32 instructions are disabled for all
device code.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libggq.so")
ARCH = os.environ.get("GGQ_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-command-line-argument",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{err}")
    return err


# Per-source flags.  The decode GEMVs keep MFMA results in ordinary VGPRs: their
# few accumulators are rescaled by the vector units after every block, and with
# AGPR results each rescale first needed a v_accvgpr_read.  It also asks a work
# counter with one atomic from one lane while the next unit's loads are in
# flight; the atomic optimiser rewrites that atomic into a wave-wide form whose
# result is read back at once, and since the load counter drains in order that
# read waited for the whole prefetch before the current unit's compute.
FILE_FLAGS = {
    "gemv_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form",
                      "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
    "gemv_ks.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(OBJ, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)))
    with ThreadPoolExecutor(max(1, jobs)) as ex:
        outs = list(ex.map(
            lambda so: _run([HIPCC, *CFLAGS, *FILE_FLAGS.get(os.path.basename(so[0]), []),
                             "-c", so[0], "-o", so[1]]),
            zip(srcs, objs)))
    if verbose:
        for o in outs:
            if o.strip():
                print(o, file=sys.stderr)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
