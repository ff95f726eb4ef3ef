"""Build the HIP library librelpos_attn.so for gfx950 (in-tree).

Every source is compiled with hipcc for gfx950 only.  Packed-fp32 VALU
instructions are disabled (``-packed-fp32-ops``); the host pass prints a
harmless warning that it does not know that feature.  MFMA results are kept
in ordinary VGPRs (``-amdgpu-mfma-vgpr-form``), which removes the copies
between accumulation and architectural registers around every MFMA.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "librelpos_attn.so")

SOURCES = [
    "api.cpp",
    "proj.hip",
    "prep.hip",
    "attn_fwd.hip",
    "attn_bwd_f32.hip",
    "attn_bwd_f16.hip",
    "attn_bwd_bf16.hip",
    "contract.hip",
]

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs (gfx950 allows it): no AGPR copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I" + os.path.join(ROOT, "include"), "-I" + SRC,
    "-Wall", "-Wno-unused-function",
]


# Sources compiled without the VGPR-form option: with it, the fp32 backward
# kernels make this compiler crash (in its pass that rewrites AGPR copies of
# MFMA results); they keep the default AGPR accumulators, which changes
# register use only, not results.
AGPR_FORM = {"attn_bwd_f32.hip"}


def flags_for(src):
    if src in AGPR_FORM:
        i = FLAGS.index("-amdgpu-mfma-vgpr-form")
        return FLAGS[:i - 1] + FLAGS[i + 1:]
    return FLAGS


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return exe


def _compile(src):
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *flags_for(src), "-c", os.path.join(SRC, src), "-o", out]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    log = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{log}")
    return out, log


def build(jobs=None, verbose=False):
    """Compile every source and link ``librelpos_attn.so``; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for (o, log) in results:
            if log.strip():
                print(f"[{os.path.basename(o)}]\n{log}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
