"""Compile the HIP sources of the attention library into ``libfa.so`` (gfx950).

Objects are built in parallel with hipcc, then linked into a shared library that
sits next to this file, where the Python binding loads it from.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
# ceiling probes (sustained matrix-core rate, HBM read bandwidth): a separate library
PROBE_LIB = os.path.join(PKG, "libfa_probe.so")
PROBE_SOURCES = ["fa_probe.hip"]
SOURCES = ["fa_fwd.hip", "fa_decode.hip", "fa_bwd.hip", "fa_fwd_fp8.hip", "fa_ffn.hip", "fa_api.hip"]
# The kernel sources assume finite inputs (non-finite Q/K/V are unsupported), which
# lets the compiler drop NaN canonicalisation around the softmax max. The C ABI source
# keeps IEEE semantics for its argument checks (isfinite(scale)).
KERNEL_ONLY_FLAGS = {"fa_fwd.hip": ["-fno-honor-nans"], "fa_decode.hip": ["-fno-honor-nans"],
                     "fa_fwd_fp8.hip": ["-fno-honor-nans"]}
ARCH = "gfx950"
# libraries the attention library links besides the HIP runtime (none)
EXTRA_LIBS = []

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the attention library needs ROCm's hipcc to build")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link libfa.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs, cmds = [], []
    for src in SOURCES + PROBE_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        if src in SOURCES:
            objs.append(obj)
        cmds.append([hipcc, *HIPCC_FLAGS, *KERNEL_ONLY_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(len(cmds)) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp, *EXTRA_LIBS])
    os.replace(tmp, LIB)
    probe_objs = [os.path.join(BUILD, src.replace(".hip", ".o")) for src in PROBE_SOURCES]
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *probe_objs, "-o", PROBE_LIB + ".tmp"])
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
