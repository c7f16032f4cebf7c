"""Build libsolattn.so in-tree with hipcc for gfx950, and the plain C example.

    python -m block_sparse_attention_14_amd.build [-v]

Every HIP source is compiled with packed-fp32 code generation disabled; the
library links only the HIP runtime. csrc/example_c.c, a C99 caller of the
library's C ABI, is compiled with the host C compiler into sol_attn_example
beside the library (found through an $ORIGIN run path).
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
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsolattn.so")
EXAMPLE = os.path.join(PKG, "sol_attn_example")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SOURCES = ["pool.hip", "plan.hip", "fwd.hip", "masks.hip", "api.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libsolattn.so")
    return path


def build(verbose: bool = False) -> str:
    """Compile every source to an object, link the shared library, return its path."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="solattn_build_") as tmp:
        objs = []
        procs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [cc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        failed = []
        for src, cmd, pr in procs:
            out, _ = pr.communicate()
            lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
            if pr.returncode != 0:
                failed.append((src, "\n".join(lines)))
            elif verbose and lines:
                print("\n".join(lines))
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n\n".join(f"[{s}]\n{o}" for s, o in failed))
        tmp_lib = LIB + ".tmp"
        link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(link), flush=True)
        r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout)
        os.replace(tmp_lib, LIB)
    build_example(verbose)
    return LIB


def build_example(verbose: bool = False) -> str:
    """Compile the C example against the built library; return the binary's path."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no host C compiler found to build the C example")
    tmp_bin = EXAMPLE + ".tmp"
    cmd = [cc, "-O2", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", INCLUDE, "-I", os.path.join(ROCM, "include"),
           os.path.join(CSRC, "example_c.c"), "-o", tmp_bin,
           "-L", PKG, "-lsolattn", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("C example build failed:\n" + r.stdout)
    os.replace(tmp_bin, EXAMPLE)
    return EXAMPLE


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
