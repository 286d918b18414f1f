"""Build libtwotower_attn.so in-tree with hipcc for gfx950.

    python -m attention_eq_block_amd.build            # library only
    python -m attention_eq_block_amd.build --asm DIR  # also dump gfx950 assembly

The library is compiled from ``csrc/`` (HIP kernels + the C-ABI host layer);
``include/twotower_attn.h`` is its public header.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtwotower_attn.so")

SOURCES = ["api.cpp", "attn_bf16.hip", "attn_f32.hip", "kv_append.hip", "merge.hip", "unmask.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    "-I", INCLUDE, "-I", CSRC,
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the register allocator then keeps operands and
    # prefetched tiles in AGPRs instead of spilling
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # schedule for memory clauses: the attention kernel's spills drop from 48 to 3 registers and its
    # call time by 1-7% on the loop, long and ragged workloads (A/B in one process)
    "-mllvm", "-amdgpu-sched-strategy=max-memory-clause",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)


def build(out: str = LIB, jobs: int = 0, extra=(), link_extra=()) -> str:
    """Compile every source to an object in parallel, then link the shared library. ``extra`` adds
    compiler flags (the sanitizer test builds a host-instrumented copy elsewhere with it)."""
    with tempfile.TemporaryDirectory(prefix="tt_build_") as tmp:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
            cmd = [HIPCC, *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
            objs.append(obj)
        failed = []
        for cmd, pr in procs:
            _, err = pr.communicate()
            noise = "is not a recognized feature for this target"
            err = "\n".join(l for l in err.splitlines() if noise not in l)
            if pr.returncode != 0:
                failed.append(f"{' '.join(cmd)}\n{err}")
            elif err.strip():
                print(err, file=sys.stderr)
        if failed:
            raise RuntimeError("HIP build failed:\n" + "\n\n".join(failed))
        tmp_out = out + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp_out])
        os.replace(tmp_out, out)
    return out


def dump_asm(outdir: str) -> None:
    os.makedirs(outdir, exist_ok=True)
    for src in SOURCES:
        if not src.endswith(".hip"):
            continue
        base = os.path.join(outdir, os.path.splitext(src)[0])
        _run([HIPCC, *COMMON, "-x", "hip", "--offload-device-only", "-S", os.path.join(CSRC, src),
              "-o", base + ".s"])


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None)
    args = ap.parse_args()
    print(build(), file=sys.stderr)
    if args.asm:
        dump_asm(args.asm)
