"""Compile libkvq.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures
import hashlib
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libkvq.so")
# sha256 of the sources the library was built from, written beside it
HASH_PATH = LIB_PATH + ".srchash"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU ops stay off (hipcc's host pass warns about the
    # unknown feature; that is harmless)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]

# per-file extra flags: the write path must round every fp32 op on its own
# Decode kernels: -fno-honor-nans, because they produce no NaN (masks use
# -inf, every inf - inf is guarded) and without NaN semantics an fmaxf of an
# MFMA result needs no canonicalising v_max first.
SOURCES = {
    "kvq_api.hip": [],
    "kvq_append.hip": ["-ffp-contract=off"],
    # keep MFMA accumulators in VGPRs: the softmax rescale touches them with
    # VALU ops, and AGPR placement costs a copy per access
    "kvq_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
    # head_dim 512: the accumulators need the AGPR half of the register file
    "kvq_decode512.hip": ["-fno-honor-nans"],
    "kvq_extend.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
    "kvq_shared.hip": ["-fno-honor-nans"],
}


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def source_hash() -> str:
    """sha256 over every file libkvq.so is built from (csrc/ and include/,
    names and contents) and the build flags."""
    flags = [x for x in COMMON if not x.startswith("-I")]   # not the tree's absolute paths
    h = hashlib.sha256(repr((flags, SOURCES)).encode())
    for d in (CSRC, INCLUDE):
        for name in sorted(os.listdir(d)):
            if name.endswith((".hip", ".h")):
                h.update(name.encode() + b"\0")
                with open(os.path.join(d, name), "rb") as f:
                    h.update(f.read())
    return h.hexdigest()


def _compile(name: str) -> str:
    src = os.path.join(CSRC, name)
    obj = os.path.join(BUILD_DIR, name + ".o")
    cmd = [HIPCC] + COMMON + SOURCES[name] + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (name, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB_PATH)
    with open(HASH_PATH, "w") as f:
        f.write(source_hash() + "\n")
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


HARNESS_SRC = os.path.join(ROOT, "tests", "convert_harness.hip")
HARNESS_LIB = os.path.join(ROOT, "tests", "libconvert_harness.so")


def harness_hash() -> str:
    """The library sources' hash extended by the conversion test harness."""
    h = hashlib.sha256(source_hash().encode())
    with open(HARNESS_SRC, "rb") as f:
        h.update(f.read())
    return h.hexdigest()


def build_test_harness(verbose: bool = False) -> str:
    """The GPU test harness that runs the append's group encoders over
    arbitrary inputs (tests/convert_harness.hip; test infrastructure, not
    part of libkvq)."""
    tmp = HARNESS_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + COMMON + ["-ffp-contract=off", "-shared", HARNESS_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for convert_harness.hip:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, HARNESS_LIB)
    with open(HARNESS_LIB + ".srchash", "w") as f:
        f.write(harness_hash() + "\n")
    if verbose:
        print("built", HARNESS_LIB)
    return HARNESS_LIB


BENCH_CLOCK_SRC = os.path.join(ROOT, "bench_clock.hip")
BENCH_CLOCK_LIB = os.path.join(ROOT, "bench_clock.so")


def build_bench_clock(verbose: bool = False) -> str:
    """The shader-clock sampler bench.py --clock-trace loads (measurement
    only, not part of libkvq)."""
    tmp = BENCH_CLOCK_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + COMMON + ["-shared", BENCH_CLOCK_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for bench_clock.hip:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, BENCH_CLOCK_LIB)
    if verbose:
        print("built", BENCH_CLOCK_LIB)
    return BENCH_CLOCK_LIB


if __name__ == "__main__":
    build(verbose=True)
    build_bench_clock(verbose=True)
    build_test_harness(verbose=True)
