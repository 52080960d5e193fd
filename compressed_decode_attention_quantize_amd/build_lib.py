"""Build libtq.so (HIP, gfx950) in-tree with hipcc.

Every HIP translation unit is compiled with packed-fp32 instructions turned
off and with correctly rounded fp32 division/sqrt; the append kernel also
with -ffp-contract=off (its arithmetic is fixed bit for bit by the format),
as is the matrix-core decode unit, which inlines the one-position quantiser
for the fused serving step (its decode code re-enables contraction with a
pragma after that include).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtq.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fhip-fp32-correctly-rounded-divide-sqrt",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]
UNITS = [
    ("tq_host.cpp", []),
    ("tq_quant.hip", ["-ffp-contract=off"]),
    ("tq_quant_tree.hip", ["-ffp-contract=off"]),
    ("tq_decode.hip", []),
    ("tq_decode_mfma.hip", ["-fno-honor-nans", "-ffp-contract=off"]),
    ("tq_decode_reg.hip", ["-fno-honor-nans", "-ffp-contract=off"]),
    ("tq_decode_q8.hip", ["-fno-honor-nans", "-ffp-contract=off"]),
    ("tq_dequant.hip", []),
    ("tq_stream.hip", []),
    ("tq_scratch.hip", []),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every unit (in parallel) and link libtq.so (always rebuilds)."""
    import concurrent.futures as cf
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src, extra in UNITS:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append((obj, [HIPCC, *COMMON, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "0")) or (os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=workers) as pool:
        outs = list(pool.map(lambda j: _run(j[1]), jobs))
    if verbose:
        for out in outs:
            if out.strip():
                print(out)
    objs = [obj for obj, _ in jobs]
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
