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


def _compile(src: str, obj: str, verbose: bool) -> None:
    cmd = [_hipcc(), "--offload-arch=gfx950", *COMMON_FLAGS, *DEVICE_FLAGS,
           "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libs5.so next to this file."""
    with tempfile.TemporaryDirectory(prefix="s5build_") as tmp:
        objs = [os.path.join(tmp, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            futs = [ex.submit(_compile, s, o, verbose) for s, o in zip(SOURCES, objs)]
            for f in futs:
                f.result()
        out_tmp = os.path.join(tmp, LIB_NAME)
        cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out_tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        shutil.copyfile(out_tmp, LIB_PATH + ".tmp")
        os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
