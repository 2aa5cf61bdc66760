"""Build the HIP library ``libkda.so`` for gfx950 with hipcc (in-tree).

Usage: ``python -m gated_delta_rule_64_amd.build`` (or ``build()`` from Python).
Every source is compiled with packed-fp32 instructions disabled for the device.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkda.so")
# measurement helper for the benchmark (a matrix-core loop), built beside the library
CEILING_LIB = os.path.join(PKG, "libkda_ceiling.so")
CEILING_SOURCE = "ceiling.hip"
SOURCES = ["kda_api.cpp", "kda_recurrent.hip", "kda_chunk.hip", "kda_chunk_bwd.hip",
           "kda_noalloc.hip"]
ARCH = os.environ.get("KDA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            "-Wno-unused-command-line-argument", "-Wno-pass-failed"]


def build(verbose: bool = False, jobs: int = 3) -> str:
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="kda_build_")
    try:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            cmd = [cc, *flags(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
            if len(procs) >= jobs:
                _wait(procs.pop(0))
        for p in procs:
            _wait(p)
        out_tmp = LIB + ".tmp%d" % os.getpid()
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp]
        subprocess.run(cmd, check=True)
        os.replace(out_tmp, LIB)
        out_tmp = CEILING_LIB + ".tmp%d" % os.getpid()
        # accumulators in VGPRs: the default AGPR form rotated the loop's accumulators
        # through copies (and measured half the matrix-core rate)
        cmd = [cc, *flags(), "-mllvm", "-amdgpu-mfma-vgpr-form", "-x", "hip", "-shared",
               os.path.join(CSRC, CEILING_SOURCE), "-o", out_tmp]
        _wait((CEILING_SOURCE, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        os.replace(out_tmp, CEILING_LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


def _wait(item):
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    # the host pass does not know the device-only target feature; drop that notice
    text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        sys.stderr.write(text + "\n")
        raise RuntimeError(f"hipcc failed on {src}")
    if text.strip():
        sys.stderr.write(text + "\n")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
