"""Build libtt.so (the HIP C-ABI library) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtt.so")
# measurement probes (a plain streaming read, the benchmark's bandwidth ceiling; the matrix-core
# rate; the attention tile loop's LDS and matrix/vector core), a library of their own so that
# they are not part of libtt's interface
PROBE_SRCS = [os.path.join(CSRC, "probe", "stream_read.hip"), os.path.join(CSRC, "probe", "tile_core.hip")]
PROBE_LIB = os.path.join(HERE, "libttprobe.so")
BUILD = os.path.join(ROOT, "_build", "libtt")
ARCH = os.environ.get("TT_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
         # packed fp32 ALU ops off for all device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


# per-file additions: the attention kernel never sees a NaN (padding is not read, masked
# scores are -inf), so it runs with IEEE mode off to drop NaN quieting before max ops
FILE_FLAGS = {"attn_mfma.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"]}


def source_files() -> list:
    """Every file libtt.so is compiled from (kernels, internal header, the C-ABI header)."""
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h"))
                  + [os.path.join(ROOT, "include", "tt.h")])


def source_hash() -> str:
    """First 16 hex digits of the SHA-256 over the sources (names and contents, in name order);
    compiled into the library as tt_build_id() so that a stale build is refused at load."""
    import hashlib
    h = hashlib.sha256()
    for f in source_files():
        h.update(os.path.relpath(f, ROOT).encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    return h.hexdigest()[:16]


def _compile(src: str, verbose: bool, sha: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), f'-DTT_SOURCE_HASH="{sha}"',
           "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    sha = source_hash()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sha), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-shared", *PROBE_SRCS, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PROBE_SRCS}:\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
