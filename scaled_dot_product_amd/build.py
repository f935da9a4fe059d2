"""Build ``libattn.so`` (the C ABI of ``include/attn.h``) for gfx950 with hipcc.

Every translation unit is compiled for ``--offload-arch=gfx950`` only, with
the packed-fp32 instructions disabled; objects go to ``_build/`` at the
repository root and the library next to this file.  hipcc cross-compiles, so
no GPU is needed.

    python -m scaled_dot_product_amd.build [-v]
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libattn.so")

FLAGS = [
    "-x", "hip", "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]

# Kernels may assume NaN-free scores (lets max() skip NaN canonicalisation);
# the host-side argument checks must not, so attn_api.cpp is built without it.
KERNEL_FLAGS = ["-fno-honor-nans"]

# (source, extra flags, object)
UNITS = [("attn_api.cpp", [], "attn_api.o"),
         ("fwd_f32.hip", KERNEL_FLAGS, "fwd_f32.o"),
         ("decode.hip", KERNEL_FLAGS, "decode.o"),
         ("scratch.hip", [], "scratch.o"),
         ("bwd_valu.hip", KERNEL_FLAGS, "bwd_valu.o")]
for _elem, _tag in (("__bf16", "bf16"), ("_Float16", "f16")):
    for _d in (128, 64, 256):
        for _src in ("fwd_mfma", "bwd_mfma"):
            UNITS.append((f"{_src}.hip",
                          KERNEL_FLAGS + [f"-DATTN_ELEM={_elem}", f"-DATTN_D={_d}",
                                          f"-DATTN_TAG={_tag}_d{_d}"],
                          f"{_src}_{_tag}_d{_d}.o"))


def hipcc() -> str:
    path = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError(f"hipcc not found ({path})")
    return path


def _compile(unit, verbose):
    src, defs, obj = unit
    cmd = [hipcc(), *FLAGS, *defs, "-c", os.path.join(CSRC, src), "-o", os.path.join(BUILD_DIR, obj)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "unknown target feature" not in line and "packed-fp32-ops" not in line
                    and line.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src} {defs}:\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        for msg in ex.map(lambda u: _compile(u, verbose), UNITS):
            if msg and verbose:
                print(msg)
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp,
           *[os.path.join(BUILD_DIR, u[2]) for u in UNITS]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
