"""Build libtq.so (HIP, gfx950) in-tree with hipcc.

    python -m ternary_quantized_linear_absmean_amd.build

Each library source in csrc/ is compiled to an object under _build/ (in
parallel), then linked into ternary_quantized_linear_absmean_amd/libtq.so.
csrc/bench_probes.hip (reference kernels the benchmark times beside the
layer, not part of the library) becomes libtq_probes.so.  The build always
recompiles.  Importing this module loads nothing from the library.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtq.so")
# reference kernels for the benchmark's context figures; not part of libtq
PROBES_SRC = "bench_probes.hip"
PROBES_LIB = os.path.join(PKG, "libtq_probes.so")

ARCH = "gfx950"
SOURCES = ["tq_api.hip", "k_pack.hip", "k_quant.hip", "k_gemv.hip", "k_gemm.hip", "k_bwd.hip"]

# -ffp-contract=off: the quantisers' fp32 products must round on their own
# (no fused multiply-add) to match the stated expression order.  Correctly
# rounded fp32 division and square root are hipcc's default and are asked for
# explicitly.  Packed-fp32 instruction selection is switched off.
COMPILE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (is ROCm installed under /opt/rocm?)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *COMPILE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    tmp = PROBES_LIB + ".tmp"
    _run([cc, *COMPILE_FLAGS, "-shared", os.path.join(CSRC, PROBES_SRC), "-o", tmp])
    os.replace(tmp, PROBES_LIB)
    if verbose:
        print(f"built {LIB} and {PROBES_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
