"""Build libunospec.so in-tree with hipcc for gfx950.

    python -m diffusion_augmented_decoding_amd.build [--verbose] [--tuning]

Compiles every csrc/*.hip and csrc/*.cpp to an object under _build/ (in
parallel) and links them into diffusion_augmented_decoding_amd/libunospec.so.
--tuning builds libunospec_tuning.so instead (objects under _build/tuning/),
compiled with -DUNO_TUNING: that library reads the UNO_* tile and split
overrides from the environment for sweeps; libunospec.so never does.
"""

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libunospec.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-variable",
    f"-I{os.path.join(ROOT, 'include')}",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# per-file flags: the attention kernel keeps its MFMA accumulators in VGPRs
# (gfx950 MFMAs take C/D from either file), which avoids copying them through
# AGPRs around the softmax rescale
FILE_FLAGS = {
    "block_attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "is not a recognized feature for this target" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose=False, jobs=None, tuning=False):
    """Compile and link libunospec.so (libunospec_tuning.so with tuning=True);
    returns its path."""
    hipcc = _hipcc()
    bdir = os.path.join(BUILD, "tuning") if tuning else BUILD
    lib = os.path.join(PKG, "libunospec_tuning.so") if tuning else LIB
    extra = ["-DUNO_TUNING"] if tuning else []
    os.makedirs(bdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    objs = []
    cmds = []
    for s in srcs:
        o = os.path.join(bdir, os.path.basename(s) + ".o")
        objs.append(o)
        cmds.append([hipcc] + COMMON_FLAGS + extra + FILE_FLAGS.get(os.path.basename(s), []) + ["-c", s, "-o", o])
    jobs = jobs or min(8, len(cmds))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = lib + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv, tuning="--tuning" in sys.argv))
