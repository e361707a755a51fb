"""Build libm2rnn.so for gfx950 with hipcc (in-tree, no JIT cache).

Run as ``python -m matrix_state_nonlinear_amd.build`` or through
``__graft_entry__.build()``.  hipcc cross-compiles without a GPU.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libm2rnn.so")
SOURCES = ["m2rnn_api.hip", "m2rnn_gates.hip", "m2rnn_fwd.hip", "m2rnn_bwd.hip",
           "m2rnn_step.hip", "m2rnn_block.hip",
           "m2rnn_newton.hip"]
ARCH = "gfx950"

# Packed fp32 VALU instructions are switched off for every kernel.  MFMA
# accumulators live in ordinary VGPRs (the step's VALU work reads them right
# after the chain; AGPR accumulators would add a copy per element).
HIP_FLAGS = ["-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form",
             "-fno-gpu-rdc", "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source to an object (in parallel), then link the library."""
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [hipcc(), *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
        while len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait() if procs[0][1].poll() is None else None
            for _, p in procs:
                if p.poll() is None:
                    p.wait()
                    break
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out, flush=True)
    if failed:
        msg = "\n".join(f"--- {s}\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    # --no-undefined: a kernel whose host stub was not emitted fails here, not at load
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
