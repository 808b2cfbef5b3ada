"""Build of libmoe_w4.so (gfx950) with hipcc, in the package directory.

Each .hip source is compiled to an object in parallel, then linked into one
shared library. Packed fp32 VALU instructions are disabled for all device
code. The result replaces the previous library atomically.

A second library, libmoe_w4_schedcheck.so, links the same objects except the
grouped GEMMs, which are compiled with MOE_SCHED_CHECK=1 (a scheduling
barrier after each K step's loads; see moe_ffn.hip). A GPU test requires it
to give the same bits as the main library.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB_NAME = "libmoe_w4.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SCHEDCHECK_PATH = os.path.join(PKG, "libmoe_w4_schedcheck.so")
SCHEDCHECK_SOURCE = "moe_ffn.hip"
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, defines=(), suffix: str = "") -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + suffix + ".o")
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], "-I", os.path.join(PKG, "..", "include"),
           "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, path: str) -> None:
    tmp = path + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, path)


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    check_src = os.path.join(CSRC, SCHEDCHECK_SOURCE)
    jobs = jobs or min(len(srcs) + 1, 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_compile, s) for s in srcs]
        fut_check = ex.submit(_compile, check_src, ("MOE_SCHED_CHECK=1",), ".schedcheck")
        objs = [f.result() for f in futs]
        obj_check = fut_check.result()
    _link(objs, LIB_PATH)
    main_check = os.path.join(BUILD, SCHEDCHECK_SOURCE + ".o")
    _link([obj_check if o == main_check else o for o in objs], SCHEDCHECK_PATH)
    return LIB_PATH


def clean():
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    print(build())
