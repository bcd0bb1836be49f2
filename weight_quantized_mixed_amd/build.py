"""Build libqgemm.so in-tree with hipcc for gfx950.

    python -m weight_quantized_mixed_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqgemm.so")
SOURCES = ["api.hip", "pack.hip", "gemv.hip", "gemv16.hip", "mfma.hip", "mfma_dl.hip", "mfma_big.hip", "reduce.hip", "quant.hip", "gemv_mfma.hip", "gemv_mfma4.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# packed fp32 vector ops are disabled for every device pass
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the device feature flag: drop that notice only
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES]

    def compile_one(i):
        src = os.path.join(CSRC, SOURCES[i])
        return _run([HIPCC, *COMMON, *DEVICE_FLAGS, "-c", src, "-o", objs[i]])

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        outs = list(ex.map(compile_one, range(len(SOURCES))))
    tmp = LIB + ".tmp"
    outs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]))
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
