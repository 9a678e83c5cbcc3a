"""Build libbitnet_w2a8.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Each csrc/*.hip file is compiled to an object in parallel, then linked into a shared
library next to this file.  A sidecar file records a hash of the sources and flags the
library was built from, so a loader can tell a current build from a stale one.
"""
from __future__ import annotations

import concurrent.futures
import hashlib
import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libbitnet_w2a8.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
HASH_PATH = LIB_PATH + ".srchash"
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # IEEE arithmetic: no contraction into FMA, correctly rounded fp32 division.
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    # never emit packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def _flags_key() -> bytes:
    """The compile flags as they affect the code: include directories are dropped, so the
    key (and every hash below) is the same wherever the repository is checked out."""
    return " ".join(f for f in FLAGS if not os.path.isabs(f)).encode()


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".hpp")))


def source_hash() -> str:
    h = hashlib.sha256()
    for path in sources() + [os.path.join(INCLUDE, "bitnet_w2a8.h")]:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    h.update(_flags_key())
    return h.hexdigest()


def kernel_hash(*names: str) -> str:
    """Hash of the named csrc files, the shared device header and the flags: identifies
    the code of one kernel family (e.g. kernel_hash("skinny.hip"))."""
    h = hashlib.sha256()
    for name in list(names) + ["device_common.hpp"]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    h.update(_flags_key())
    return h.hexdigest()


def is_current() -> bool:
    if not os.path.exists(LIB_PATH) or not os.path.exists(HASH_PATH):
        return False
    with open(HASH_PATH) as f:
        return f.read().strip() == source_hash()


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip for gfx950 and link libbitnet_w2a8.so in-tree."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    hips = [s for s in sources() if s.endswith(".hip")]
    jobs = min(len(hips), int(os.environ.get("MAX_JOBS", "8")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, hips))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    with open(HASH_PATH, "w") as f:
        f.write(source_hash())
    if verbose:
        print(f"built {LIB_PATH}", file=sys.stderr)
    return LIB_PATH


PROBES_SRC = os.path.join(PKG_DIR, "probes", "ceilings.hip")
PROBES_LIB = os.path.join(PKG_DIR, "libbitnet_probes.so")


def build_probes(verbose: bool = False) -> str:
    """Compile the ceiling microbenchmarks (not part of the BitLinear library)."""
    tmp = PROBES_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-shared", PROBES_SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PROBES_SRC}:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, PROBES_LIB)
    if verbose:
        print(f"built {PROBES_LIB}", file=sys.stderr)
    return PROBES_LIB


if __name__ == "__main__":
    build(verbose=True)
    build_probes(verbose=True)
