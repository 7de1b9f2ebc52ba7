"""Compile the HIP sources into ``libttt_linear.so`` next to this file (gfx950).

Each translation unit is compiled in parallel with hipcc, then linked into
one shared library.  Packed-FP32 instruction selection is switched off for
all device code.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libttt_linear.so")
#: the throughput probes the benchmark measures its ceilings with (not the scan's ABI)
PEAKS_LIB = os.path.join(HERE, "libttt_peaks.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

SOURCES = ["ttt_linear.hip", "scan_valu.hip", "scan_mfma.hip", "bwd_mfma.hip", "bwd_valu.hip",
           "proj_mfma.hip", "scan_mlp_valu.hip", "scan_mlp_mfma.hip"]
PEAK_SOURCES = ["peaks.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


#: kernel names (as the library reports them) whose source file is named otherwise
KERNEL_SOURCES = {"mlp_mfma": "scan_mlp_mfma", "mlp_valu": "scan_mlp_valu"}


def source_digest(kernel: str | None = None) -> str:
    """SHA-256 identifying a build: over one kernel's source and the shared
    kernel header (``kernel`` = "scan_mfma", "bwd_mfma", "scan_valu",
    "mlp_mfma", ...), or over every source and the public header
    (``kernel`` = None)."""
    import hashlib
    h = hashlib.sha256()
    if kernel is not None:
        names = [KERNEL_SOURCES.get(kernel, kernel) + ".hip", "scan_common.h"]
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


# ---------------------------------------------------------------------------
# A check of the generated gfx950 code: no vector instruction may overwrite a
# register that an in-flight v_mfma_f32_16x16x16_bf16 reads as its
# accumulator input within SRCC_WAR_MIN wait states of that product's issue.
# Built for gfx950, such a write three to six wait states after the issue was
# read by the product (wrong results, no fault); the 16x16x32 form reads its
# accumulator input early and is not subject to this.  The 4x4x1 fp32 products
# of the serial pass are held to the same rule as a precaution (their targets
# are left alone for a whole token by construction).
# ---------------------------------------------------------------------------
SRCC_WAR_MIN = 8
_CHECKED_MFMA = ("v_mfma_f32_16x16x16_bf16", "v_mfma_f32_4x4x1_16b_f32")
_NO_VREG_DEST = ("s_", "ds_write", "ds_store", "global_store", "buffer_store", "flat_store",
                 "scratch_store")


def _vregs(text: str) -> set:
    out = set()
    for m in re.finditer(r"\b([va])\[(\d+):(\d+)\]", text):
        out.update(f"{m.group(1)}{r}" for r in range(int(m.group(2)), int(m.group(3)) + 1))
    for m in re.finditer(r"\b([va])(\d+)\b", text):
        out.add(m.group(1) + m.group(2))
    return out


def srcc_war_hazards(asm: str, min_wait: int = SRCC_WAR_MIN) -> list:
    """Places in gfx950 assembly where a non-MFMA instruction writes a register
    that an earlier checked MFMA reads as its accumulator input (and does not
    also write), fewer than ``min_wait`` wait states after that MFMA (each
    instruction counts one, ``s_nop n`` counts n + 1).  Returns
    ``(mfma line, writer line, wait states)`` tuples."""
    ins = []
    for line in asm.splitlines():
        s = line.split(";")[0].strip()
        if s and not s.startswith(".") and not s.endswith(":"):
            ins.append(s)
    found = []
    for i, s in enumerate(ins):
        op = s.split()[0]
        if op not in _CHECKED_MFMA:
            continue
        ops = s.split(None, 1)[1].split(",")
        if len(ops) < 4:
            continue
        srcc = _vregs(ops[3]) - _vregs(ops[0])
        if not srcc:
            continue
        ws = 0
        for t in ins[i + 1:]:
            if ws >= min_wait:
                break
            top = t.split()[0]
            if top == "s_nop":
                ws += int(t.split()[1], 0) + 1
                continue
            if " " in t and not top.startswith(_NO_VREG_DEST) and "mfma" not in top:
                if _vregs(t.split(None, 1)[1].split(",")[0]) & srcc:
                    found.append((s, t, ws))
                    break
            ws += 1
    return found


def build(verbose: bool = False) -> str:
    """Compile every source, link the library and the probe library; returns
    the library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    all_sources = SOURCES + PEAK_SOURCES
    objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in all_sources]
    # the digest of the sources goes into ttt_version(), so a stale library can be told apart
    digest = [f'-DTTT_SOURCE_DIGEST="{source_digest()}"']
    # -save-temps=obj keeps the device assembly each object is assembled from
    cmds = [[HIPCC, *CFLAGS, *digest, "-save-temps=obj", "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(all_sources, objs)]
    with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    bad = []
    for s in all_sources:
        asm = os.path.join(BUILD_DIR, f"{os.path.splitext(s)[0]}-hip-amdgcn-amd-amdhsa-{ARCH}.s")
        if not os.path.exists(asm):
            raise RuntimeError(f"device assembly of {s} not found at {asm}")
        with open(asm) as f:
            bad += [(s, *h) for h in srcc_war_hazards(f.read())]
    if bad:
        raise RuntimeError("accumulator-input overwrite of an in-flight 16x16x16 MFMA:\n" +
                           "\n".join(f"  {s}: {m} | {w} ({n} wait states)" for s, m, w, n in bad))
    # flat (generic-address) memory instructions count against the LDS wait
    # counter as well, so every LDS wait after one waits for its memory
    # round trip; device pointers here are global and LDS is addressed directly
    flat = []
    for s in all_sources:
        asm = os.path.join(BUILD_DIR, f"{os.path.splitext(s)[0]}-hip-amdgcn-amd-amdhsa-{ARCH}.s")
        with open(asm) as f:
            flat += [f"  {s}: {l.strip()}" for l in f if l.lstrip().startswith("flat_")]
    if flat:
        raise RuntimeError("flat memory instructions in device code:\n" + "\n".join(flat[:20]))
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", PEAKS_LIB + ".tmp",
          *objs[len(SOURCES):]])
    os.replace(PEAKS_LIB + ".tmp", PEAKS_LIB)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs[:len(SOURCES)]])
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
