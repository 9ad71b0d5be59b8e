"""Build libkvq.so (the HIP kernels and their C ABI) for gfx950, in-tree.

hipcc compiles every ``csrc/*.hip`` file to an object in parallel, then links
them into ``kv_quantization_amd/libkvq.so``.  No torch extension machinery:
the library has a plain C ABI (``include/kvq.h``) and is loaded with ctypes.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB = PKG / "libkvq.so"
BUILD_DIR = ROOT / "_build"

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",          # the quantizers are specified op by op; no silent FMA
    "-mllvm", "-amdgpu-mfma-vgpr-form",   # MFMA accumulators in VGPRs: no AGPR copies in the epilogues
    "-fno-gpu-rdc",
    # keep packed fp32 VALU forms (v_pk_fma/mul/add_f32) out of the code object
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def sources():
    return sorted(CSRC.glob("*.hip"))


def build(verbose: bool = False) -> Path:
    BUILD_DIR.mkdir(exist_ok=True)
    srcs = sources()

    def compile_one(src: Path) -> Path:
        obj = BUILD_DIR / (src.stem + ".o")
        cmd = [HIPCC, *FLAGS, "-c", str(src), "-o", str(obj)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src.name}:\n{out}")
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB.with_suffix(f".so.tmp{os.getpid()}")
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
