"""Compile the HIP libraries in-tree for gfx950.

liblso.so         the C ABI of include/lso.h (fused kernel, runtime, streams)
liblso_probes.so  measurement / verification probes (copy ceiling, BF16 cast)
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -ffp-contract=off: FMAs are spelled out in the kernel; nothing else fuses.
# -fhip-fp32-correctly-rounded-divide-sqrt: FP32 division and sqrtf round
# correctly (stated here rather than left to the compiler's default).
# Packed FP32 instructions are disabled for all device code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]

# ROCr, for copies on named SDMA engines (lso_sdma.cpp)
LINK = ["-lhsa-runtime64"]

LIBS = {
    "liblso.so": ["lso_adam.hip", "lso_copy.hip", "lso_tiled.hip", "lso_noalloc.hip", "lso_runtime.cpp",
                  "lso_stream.cpp", "lso_io.cpp", "lso_shadow.cpp", "lso_sdma.cpp"],
    "liblso_probes.so": ["lso_probes.hip", "lso_probe_io.cpp", "lso_sdma.cpp"],
}


def lib_path(name: str = "liblso.so") -> str:
    return os.path.join(HERE, name)


def build(verbose: bool = False) -> list[str]:
    out = []
    for name, srcs in LIBS.items():
        target = lib_path(name)
        tmp = target + ".tmp"
        cmd = [HIPCC, *FLAGS, *[os.path.join(CSRC, s) for s in srcs], "-o", tmp, *LINK]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        r = subprocess.run(cmd, capture_output=True, text=True)
        # the host pass does not know the packed-fp32 feature; that note is noise
        noise = "'-packed-fp32-ops' is not a recognized feature"
        err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {name}:\n{err}")
        if err.strip() and verbose:
            print(err, file=sys.stderr)
        os.replace(tmp, target)
        out.append(target)
    return out


if __name__ == "__main__":
    for p in build(verbose=True):
        print(p)
