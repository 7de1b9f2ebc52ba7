"""Compile the HIP sources into ``libttt_linear.so`` next to this file (gfx950).

Each translation unit is compiled in parallel with hipcc, then linked into
one shared library.  Packed-FP32 instruction selection is switched off for
all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libttt_linear.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

SOURCES = ["ttt_linear.hip", "scan_valu.hip", "scan_mfma.hip", "bwd_mfma.hip", "proj_mfma.hip",
           "scan_mlp_valu.hip", "scan_mlp_mfma.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def source_digest(kernel: str | None = None) -> str:
    """SHA-256 identifying a build: over one kernel's source and the shared
    kernel header (``kernel`` = "scan_mfma", "bwd_mfma", "scan_valu"), or over
    every source and the public header (``kernel`` = None)."""
    import hashlib
    h = hashlib.sha256()
    if kernel is not None:
        names = [kernel + ".hip", "scan_common.h"]
    else:
        names = sorted(os.listdir(CSRC))
    for name in names:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    if kernel is None:
        with open(os.path.join(INCLUDE, "ttt_linear.h"), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link the library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    # the digest of the sources goes into ttt_version(), so a stale library can be told apart
    digest = [f'-DTTT_SOURCE_DIGEST="{source_digest()}"']
    cmds = [[HIPCC, *CFLAGS, *digest, "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs])
    # a kernel whose host-side stub was not emitted (the host pass can drop a
    # kernel template without a diagnostic) would only fail when loaded
    undef = [l for l in _run(["nm", "-D", "--undefined-only", tmp]).splitlines()
             if "__device_stub__" in l]
    if undef:
        os.remove(tmp)
        raise RuntimeError("kernels without a host stub:\n" + "\n".join(undef))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
