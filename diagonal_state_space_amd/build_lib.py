"""Build libs5.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: python -m diagonal_state_space_amd.build_lib [-v]
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libs5.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# peak-rate probes of the roofline report (include/s5_peak.h), a library of
# their own: they measure the chip and are no part of the S5 path
PEAK_LIB_NAME = "libs5_peak.so"
PEAK_LIB_PATH = os.path.join(PKG, PEAK_LIB_NAME)
PEAK_SOURCES = ["s5_peak.hip"]

SOURCES = ["s5_api.cpp", "s5_discretize.hip", "s5_forward.hip", "s5_pack.hip", "s5_step.hip", "s5_glu.hip",
           "s5_fused_bf16_ti.hip", "s5_fused_bf16_tv.hip", "s5_fused_f32_ti.hip", "s5_fused_f32_tv.hip"]

# Packed-FP32 instructions are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
                f"-I{INCLUDE}", f"-I{CSRC}"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# per-source extra flags: the MFMA throughput probe keeps its accumulators in
# ordinary VGPRs (with AGPR accumulators the compiler rotated them through
# register moves on every loop trip, which halved the measured rate)
EXTRA_FLAGS = {"s5_peak.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, obj: str, verbose: bool) -> None:
    cmd = [_hipcc(), "--offload-arch=gfx950", *COMMON_FLAGS, *DEVICE_FLAGS, *EXTRA_FLAGS.get(src, []),
           "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)


def _link(objs, name: str, path: str, tmp: str, verbose: bool) -> None:
    out_tmp = os.path.join(tmp, name)
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out_tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    shutil.copyfile(out_tmp, path + ".tmp")
    os.replace(path + ".tmp", path)


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libs5.so (and the probes'
    libs5_peak.so) next to this file."""
    with tempfile.TemporaryDirectory(prefix="s5build_") as tmp:
        srcs = SOURCES + PEAK_SOURCES
        objs = {s: os.path.join(tmp, os.path.splitext(s)[0] + ".o") for s in srcs}
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
            futs = [ex.submit(_compile, s, objs[s], verbose) for s in srcs]
            for f in futs:
                f.result()
        _link([objs[s] for s in SOURCES], LIB_NAME, LIB_PATH, tmp, verbose)
        _link([objs[s] for s in PEAK_SOURCES], PEAK_LIB_NAME, PEAK_LIB_PATH, tmp, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
