"""Build libintattn.so in-tree for gfx950 (hipcc cross-compiles without a GPU).

    python -m integer_only_quantized_amd.build

Host derivation (intattn_host.cpp) is compiled by g++ with -ffp-contract=off
so its binary64 arithmetic matches a plain IEEE evaluation; the HIP kernels
are compiled by hipcc for gfx950 with packed-FP32 instruction selection
disabled (the kernels use no floating point; the flag is set uniformly).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libintattn.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
# roofline calibration kernels (pure MFMA / VALU loops), a separate library
PROBE_LIB_PATH = os.path.join(HERE, "libintattn_probe.so")
PROBE_SOURCES = ["peak_probe.hip"]
BUILD_DIR = os.path.join(ROOT, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-Wextra"]


def _run(cmd):
    print("+ " + " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


HOST_SOURCES = ["intattn_host.cpp", "intattn_api.cpp"]
HIP_SOURCES = ["ia_general.hip", "ia_short.hip", "ia_long.hip", "ia_decode.hip", "ia_decode_split.hip", "ia_stages.hip",
               "ia_kvcache.hip", "ia_noalloc.hip", "ia_short16.hip"]
# Per-source code-generation options: the long- and short-row kernels keep
# their MFMA accumulators in ordinary VGPRs (no accumulator-register copies
# when the scores are post-processed on the VALU).
_VGPR_MFMA = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
HIP_EXTRA = {"ia_long.hip": _VGPR_MFMA, "ia_short.hip": _VGPR_MFMA, "ia_short16.hip": _VGPR_MFMA,
             "ia_stages.hip": _VGPR_MFMA}


def build(verbose: bool = True, jobs: int = 8) -> str:
    """Compile every source (in parallel) and link libintattn.so; returns its path."""
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(BUILD_DIR, exist_ok=True)
    inc = ["-I" + INCLUDE, "-I" + CSRC]
    cxx = shutil.which("g++") or "g++"
    cmds, objs = [], []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src.rsplit(".", 1)[0] + ".o")
        cmds.append([cxx] + HOST_FLAGS + inc + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src.rsplit(".", 1)[0] + ".o")
        cmds.append([HIPCC] + HIP_FLAGS + HIP_EXTRA.get(src, []) + inc + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    probe_objs = []
    for src in PROBE_SOURCES:
        obj = os.path.join(BUILD_DIR, src.rsplit(".", 1)[0] + ".o")
        cmds.append([HIPCC] + HIP_FLAGS + inc + ["-c", os.path.join(CSRC, src), "-o", obj])
        probe_objs.append(obj)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(_run, cmds))
    for objects, path in ((objs, LIB_PATH), (probe_objs, PROBE_LIB_PATH)):
        tmp = path + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objects + ["-o", tmp])
        os.replace(tmp, path)
    return LIB_PATH


if __name__ == "__main__":
    build()
    sys.exit(0)
