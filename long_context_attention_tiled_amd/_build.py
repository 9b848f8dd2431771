"""Build ``libattn.so`` (HIP kernels + C ABI) for gfx950 with hipcc.

Every ``csrc/*.hip`` file is compiled to an object in ``_build/`` (in
parallel), then linked into ``libattn.so`` next to this file.  Packed fp32
VALU instructions are disabled for all device code.

The library carries the hash of the sources and flags it was built from
(``attn_build_id``); the loader refuses a library whose hash differs from
that of the sources next to it, so a stale build is never tested or timed.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import hashlib
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build", "libattn")
LIB = os.path.join(PKG, "libattn.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def source_files() -> list[str]:
    """Every file the library is compiled from: csrc/*.hip, csrc/*.h, include/*.h."""
    files = glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h"))
    files += glob.glob(os.path.join(ROOT, "include", "*.h"))
    return sorted(files)


def source_hash() -> str:
    """sha256 (first 16 hex digits) over the library's sources and compile flags."""
    h = hashlib.sha256()
    for f in source_files():
        with open(f, "rb") as fh:
            h.update(os.path.relpath(f, ROOT).encode() + b"\0" + fh.read() + b"\0")
    h.update(" ".join(HIPCC_FLAGS).encode())
    return h.hexdigest()[:16]


def _hipcc() -> str:
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: ROCm is required to build libattn")


def _compile(src: str, obj: str, hipcc: str, build_id: str) -> None:
    cmd = [hipcc, *HIPCC_FLAGS, f'-DLCAT_BUILD_ID="{build_id}"', "-I", os.path.join(ROOT, "include"),
           "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{r.stderr}")


def build(jobs: int | None = None, verbose: bool = True) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    build_id = source_hash()
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, s, o, hipcc, build_id) for s, o in zip(srcs, objs)]
        for f in futs:
            f.result()
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} (sources {build_id})")
    return LIB


if __name__ == "__main__":
    build()
