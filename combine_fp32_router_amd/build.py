"""Build ``libmoe_route.so`` and ``libmoe_harness.so`` (gfx950) in-tree with hipcc.

``libmoe_route.so`` is the product: the data path's kernels and the C ABI of
``include/moe_route.h`` and ``include/moe_recv.h``.  ``libmoe_harness.so`` is
test support (``include/moe_harness.h``): the expert and exchange stand-ins
and the bandwidth probes; it does not link the product library.  Every
source is compiled separately, in parallel.  Flags:
  --offload-arch=gfx950      CDNA4 only
  -O3 -ffp-contract=off      only the explicit fmaf() calls fuse; the int8
                             divide/round and the stand-in multiply stay the
                             single IEEE operations the format defines
  -target-feature -packed-fp32-ops  keep the compiler from emitting packed
                             fp32 (v_pk_*_f32) instructions
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libmoe_route.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
HARNESS_PATH = os.path.join(HERE, "libmoe_harness.so")

SOURCES = ["route_topk.hip", "dispatch_layout.hip", "dispatch_pack.hip", "combine.hip",
           "recv_regroup.hip", "combine_pack.hip", "static_scratch.hip", "abi.cpp"]
HARNESS_SOURCES = ["harness.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *lang, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in (r.stderr or "").splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def _link(objs, path: str, verbose: bool) -> str:
    tmp = path + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(path)} failed:\n{r.stderr}")
    os.replace(tmp, path)
    return path


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link both libraries; returns the product
    library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + HARNESS_SOURCES
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in HARNESS_SOURCES], HARNESS_PATH, verbose)
    return _link([objs[s] for s in SOURCES], LIB_PATH, verbose)


def clean() -> None:
    shutil.rmtree(BUILD_DIR, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
