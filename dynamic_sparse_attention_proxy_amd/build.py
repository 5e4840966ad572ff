"""Build the CRISP HIP library (libcrisp.so) for gfx950, in-tree.

Usage: python -m dynamic_sparse_attention_proxy_amd.build  [--jobs J]
Objects go to _build/ at the repository root; the shared library lands next
to this file, where the binding loads it.
"""
import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcrisp.so")
SOURCES = ["api.hip", "proxy.hip", "select.hip", "attn.hip", "jsd.hip", "cols.hip"]
# Measurement probe, a library of its own so it stays out of the CRISP ABI.
PROBE_LIB = os.path.join(PKG, "libcrisp_probe.so")
PROBE_SOURCES = ["probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-command-line-argument",
    "-Wno-inline-asm",  # the LDS-DMA asm names m0, which it sets itself
    # packed fp32 ops stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
]


# Kernel sources may assume finite floats (fmaxf then maps to v_max3 with no
# canonicalisation); the host-side argument validation in api.hip must see
# NaNs, so it is built without the flag.
KERNEL_ONLY_FLAGS = ["-fno-honor-nans"]
HOST_VALIDATION_SOURCES = ("api.hip",)


# The attention kernel wraps each (head, query block) item in a loop over
# claimed items.  Machine-level loop-invariant code motion would hoist the
# constants of an item's prologue and epilogue out of that loop and hold them
# in scalar registers across the item's main loop, which then spills; the
# main loop itself gains nothing from it (its invariants are written outside
# it already).
PER_SOURCE_FLAGS = {"attn.hip": ["-mllvm", "-disable-machine-licm"]}


def flags_for(src):
    return (FLAGS + ([] if src in HOST_VALIDATION_SOURCES else KERNEL_ONLY_FLAGS)
            + PER_SOURCE_FLAGS.get(src, []))


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + flags_for(src) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    return src, obj, r.returncode, out


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        print(r.stdout + r.stderr, file=sys.stderr)
        raise RuntimeError(f"link of {os.path.basename(out)} failed")
    os.replace(tmp, out)


def build(jobs: int = 4, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        results = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    objs = {}
    for src, obj, rc, out in results:
        if out.strip() and (verbose or rc != 0):
            print(f"[{src}]\n{out}", file=sys.stderr)
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {src}")
        objs[src] = obj
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))
