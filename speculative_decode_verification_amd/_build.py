"""Build libsdv.so (and the synthetic-input fill library) in-tree with hipcc for gfx950."""

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libsdv.so")
SYNTH_LIB_PATH = os.path.join(ROOT, "synth", "libsdvsynth.so")

ARCH = "gfx950"
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-fvisibility=hidden",
    # keep the compiler from emitting packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
LIB_SOURCES = ["api.hip", "q4_matvec.hip", "q4_dense.hip", "moe_experts.hip", "route.hip", "combine.hip", "gdn.hip",
               "accept.hip", "gdn_prep.hip"]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libsdv")
    return path


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops" not in l)  # host-pass notice about the device-only feature
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build_library(verbose=False):
    """Compile every kernel source and link libsdv.so next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in LIB_SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        outs = list(ex.map(_run, cmds))
    tmp = LIB_PATH + ".tmp"
    outs.append(_run([cc, *HIPCC_FLAGS, "-shared", *objs, "-o", tmp]))
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("\n".join(o for o in outs if o.strip()))
    return LIB_PATH


def build_synth(verbose=False):
    """Compile the device fill used to generate large synthetic weight banks."""
    cc = hipcc()
    src = os.path.join(ROOT, "synth", "fill.hip")
    tmp = SYNTH_LIB_PATH + ".tmp"
    out = _run([cc, *HIPCC_FLAGS, "-shared", src, "-o", tmp])
    os.replace(tmp, SYNTH_LIB_PATH)
    if verbose and out.strip():
        print(out)
    return SYNTH_LIB_PATH


def build_all(verbose=False):
    return build_library(verbose), build_synth(verbose)


if __name__ == "__main__":
    print(build_all(verbose=True))
