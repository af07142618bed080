"""Build the plain-C consumer of the layer's C ABI (clr_c_driver.c) with gcc.

Test infrastructure: the program links the in-tree libclr.so and the HIP
runtime, and includes only include/clr.h and the HIP runtime API header, so
compiling it as C11 also checks that the public header is plain C.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "clr_c_driver.c")
OUT = os.path.join(HERE, "_build", "clr_c_driver")
PKG = os.path.join(ROOT, "chunked_linear_recurrence_chunk_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out: str = OUT) -> str:
    """Compile (always) and return the executable's path."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), SRC, "-o", tmp,
           "-L", PKG, "-lclr", "-Wl,-rpath,$ORIGIN/" + os.path.relpath(PKG, os.path.dirname(out)),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("gcc failed for %s:\n%s" % (SRC, p.stderr))
    os.replace(tmp, out)
    return out


def path() -> str:
    """The built executable, building it first if absent."""
    return OUT if os.path.exists(OUT) else build()
