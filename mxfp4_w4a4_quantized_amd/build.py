"""Build step for the HIP library ``libmxfp4.so`` (gfx950 only).

Compiles the kernels and the C-ABI layer in ``csrc/`` with hipcc into a shared
library next to this file, and the benchmark's MFMA-rate measurement kernel
(``csrc/ceiling.hip``) into ``libmxfp4_ceiling.so``.  Flags:
  --offload-arch=gfx950          CDNA4 only
  -ffp-contract=off              no implicit fused multiply-adds: the quantizer's
                                 fp32 results follow the written op order
  -target-feature -packed-fp32-ops  no packed fp32 VALU instructions
  -fvisibility=hidden            only the C-ABI symbols are exported
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmxfp4.so")
CEILING_LIB = os.path.join(HERE, "libmxfp4_ceiling.so")
SOURCES = ["api.cpp", "quantize.hip", "gemm.hip", "gemm_large.hip", "gemm_small.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I" + INCLUDE, "-I" + CSRC,
]


def build(verbose: bool = False, jobs: int = 3) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [HIPCC] + FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature; harmless
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if p.returncode != 0 or (verbose and lines):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed for " + ", ".join(failed))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    # the measurement kernel, a library of its own (not part of the MXFP4 ABI)
    cmd = [HIPCC] + FLAGS + ["-shared", os.path.join(CSRC, "ceiling.hip"), "-o", CEILING_LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        print(r.stdout.decode(errors="replace"), file=sys.stderr)
        raise RuntimeError("hipcc failed for ceiling.hip")
    os.replace(CEILING_LIB + ".tmp", CEILING_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
