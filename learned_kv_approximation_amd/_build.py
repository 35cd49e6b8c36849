"""Builds libkva.so (the HIP kernels and the C ABI) for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkva.so")
SOURCES = ["kva_runtime.hip", "kva_gemm.hip", "kva_attn.hip", "kva_misc.hip", "kva_deltanet.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


# Per-source code-generation options.  The attention kernel keeps its MFMA
# accumulators in ordinary VGPRs: with them in AGPRs the compiler copies the
# output accumulator between the two register files around the softmax
# rescale every tile (about 200 extra moves per tile; measured 6-7% slower).
EXTRA = {"kva_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def compile_command(src: str, obj: str) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # packed fp32 VALU ops stay off: the compiler would form them from
            # scalar float code, and the path does not rely on them
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            *EXTRA.get(src, []),
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            "-c", os.path.join(CSRC, src), "-o", obj]


def link_command(objs: list, out: str = LIB) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out]


def _run(cmds: list) -> str:
    """Runs the commands concurrently; raises with the first failure's output."""
    noise = "not a recognized feature for this target"
    procs = [(c, subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)) for c in cmds]
    errs = []
    for c, p in procs:
        _, err = p.communicate()
        err = "\n".join(l for l in (err or "").splitlines() if noise not in l)
        if p.returncode != 0:
            for _, q in procs:
                q.wait()
            raise RuntimeError("hipcc failed:\n" + " ".join(c) + "\n" + err)
        errs.append(err)
    return "\n".join(e for e in errs if e.strip())


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libkva.so (always recompiles)."""
    tmp = LIB + ".tmp"
    with tempfile.TemporaryDirectory(prefix="kva_build_") as d:
        objs = [os.path.join(d, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        err = _run([compile_command(s, o) for s, o in zip(SOURCES, objs)])
        err += _run([link_command(objs, tmp)])
    if verbose and err.strip():
        print(err)
    os.replace(tmp, LIB)
    return LIB
