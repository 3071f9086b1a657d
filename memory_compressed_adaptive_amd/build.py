"""Builds the package's native libraries in-tree with hipcc for gfx950.

    python -m memory_compressed_adaptive_amd.build

libmicroadam.so  -- the MicroAdam step (C ABI in include/microadam.h)
libmasynth.so    -- the seeded synthetic-input generator used by the benchmark
                    and the tests (no optimizer arithmetic in it)

Floating point: no contraction (fp32 results must equal the CPU oracle's one
rounding per operation), correctly rounded fp32 division and square root,
denormals kept, and no packed-fp32 instructions.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unused-function", "-Wno-unused-value",
    f"-I{INCLUDE}", f"-I{CSRC}",
]

TARGETS = {
    "libmicroadam.so": [os.path.join(CSRC, "microadam.hip")],
    "libmasynth.so": [os.path.join(CSRC, "synth.hip")],
}


def build(verbose: bool = False, only: str | None = None) -> list[str]:
    out = []
    for name, srcs in TARGETS.items():
        if only and name != only:
            continue
        dst = os.path.join(PKG, name)
        tmp = dst + ".tmp"
        cmd = [HIPCC, *COMMON, *srcs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed for {name}")
        elif verbose and (r.stderr.strip()):
            # hipcc's host pass does not know the packed-fp32 feature; harmless
            lines = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
            if any(ln.strip() for ln in lines):
                sys.stderr.write("\n".join(lines) + "\n")
        os.replace(tmp, dst)
        out.append(dst)
    return out


if __name__ == "__main__":
    for p in build(verbose="-v" in sys.argv):
        print(p)
