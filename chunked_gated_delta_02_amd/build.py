"""Build libgdr.so (HIP, gfx950) in-tree with hipcc.

The library is compiled from ``csrc/*.hip`` and ``csrc/gdr_api.cpp`` into
``chunked_gated_delta_02_amd/libgdr.so``.  The same sources compiled with
``-DGDR_DEBUG_DELAY`` give ``libgdr_delay.so``, the race-test build whose
barriers can delay chosen waves (include/libgdr_debug.h); only tests load it.  After linking, the build checks
that the shared object carries a gfx950 code object and that every kernel
was compiled with non-trivial register usage (an empty kernel body is the
signature of a build that silently dropped the target architecture).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libgdr.so")
DELAY_LIB = os.path.join(HERE, "libgdr_delay.so")
# device code without kernels (the static workspace of the allocation-free
# entry point): exempt from the check that every .hip file compiled kernels
NO_KERNEL_SOURCES = {"gdr_noalloc.hip"}
# measurement probes (peak MFMA rate, streaming bandwidth): their own library
PROBE_LIB = os.path.join(HERE, "libgdr_probe.so")
PROBE_SOURCES = ["gdr_probe.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["gdr_fwd.hip", "gdr_bwd.hip", "gdr_api.cpp", "gdr_noalloc.hip", "gdr_rmsnorm.hip"]
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU instructions are kept off for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]


def _compile(src: str, verbose: bool, delay: bool = False) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + (".delay.o" if delay else ".o"))
    cmd = [HIPCC] + FLAGS + (["-DGDR_DEBUG_DELAY"] if delay else []) + [
        "-c", os.path.join(CSRC, src), "-o", obj, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr[-8000:]))
    _check_resources(src, r.stderr)
    if verbose:
        print(r.stderr)
    return obj


def _check_resources(src: str, remarks: str) -> None:
    names = re.findall(r"Function Name: (\S+)", remarks)
    vgprs = [int(x) for x in re.findall(r"VGPRs: (\d+)", remarks)]
    if src.endswith(".hip") and src not in NO_KERNEL_SOURCES:
        if not names:
            raise RuntimeError("no kernels were compiled for %s (target dropped?)" % src)
        for n, v in zip(names, vgprs):
            if v < 4:
                raise RuntimeError("kernel %s in %s has %d VGPRs: empty body?" % (n, src, v))


def _check_arch(lib: str) -> None:
    with open(lib, "rb") as f:
        blob = f.read()
    if ("amdgcn-amd-amdhsa--" + ARCH).encode() not in blob and ARCH.encode() not in blob:
        raise RuntimeError("%s carries no %s code object" % (lib, ARCH))


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr[-8000:])
    _check_arch(tmp)
    os.replace(tmp, lib)


def build(verbose: bool = False, delay: bool = True) -> str:
    """Build libgdr.so, the probe library libgdr_probe.so and (delay=True)
    the race-test build libgdr_delay.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = ([(s, False) for s in SOURCES] + [(s, False) for s in PROBE_SOURCES] +
            ([(s, True) for s in SOURCES] if delay else []))
    with cf.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1]), jobs))
    n, m = len(SOURCES), len(PROBE_SOURCES)
    _link(objs[:n], LIB)
    _link(objs[n:n + m], PROBE_LIB)
    if delay:
        _link(objs[n + m:], DELAY_LIB)
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD_DIR, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose=False))
