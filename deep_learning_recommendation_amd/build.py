"""Build libdlrm.so (and the synthetic-table filler libsynth.so) for gfx950.

Every HIP source is compiled with hipcc for gfx950 only, with packed fp32
instructions disabled and floating-point contraction off (the bit-exact
kernels rely on separate fp32 adds and multiplies), then linked into a
shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
]

LIBDLRM_SOURCES = ["abi.hip", "embbag.hip", "interact.hip", "gemm.hip", "mlp.hip", "sparse.hip"]


def _compile(src: str, obj: str) -> None:
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build_library(name: str, srcs, out: str, jobs: int = 8) -> str:
    os.makedirs(os.path.join(BUILD_DIR, name), exist_ok=True)
    objs = [os.path.join(BUILD_DIR, name, os.path.basename(s) + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        list(ex.map(_compile, srcs, objs))
    _link(objs, out)
    return out


def build_all(jobs: int = 8) -> list:
    csrc = os.path.join(HERE, "csrc")
    libdlrm = build_library("dlrm", [os.path.join(csrc, s) for s in LIBDLRM_SOURCES],
                            os.path.join(HERE, "libdlrm.so"), jobs)
    synth_src = os.path.join(ROOT, "synth", "csrc", "fill_tables.hip")
    libsynth = build_library("synth", [synth_src], os.path.join(ROOT, "synth", "libsynth.so"), jobs)
    return [libdlrm, libsynth]


if __name__ == "__main__":
    for p in build_all():
        print(p)
