"""Host-sanitizer build of the C ABI's argument validation.

Compiles the library sources with AddressSanitizer and UndefinedBehaviorSanitizer on the
host side only (device code is compiled as usual), links them with clang++ into
``_build/sanitize/libfa_san.so`` and builds the host-only driver ``csrc/fa_abi_check.cpp``
against it. Running the driver exercises every validation path of the C ABI without a
GPU; any sanitizer report or refused check makes it fail.
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

from . import build as _b

OUT = os.path.join(_b.BUILD, "sanitize")
LIB = os.path.join(OUT, "libfa_san.so")
DRIVER = os.path.join(OUT, "fa_abi_check")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
# host-side sanitizers only: each -fsanitize= follows -Xarch_host on the hipcc lines
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
LINK_SAN = ["-fsanitize=address,undefined", "-shared-libsan"]


def build_sanitized() -> str:
    """Build the sanitized library and the validation driver; returns the driver's path."""
    hipcc = _b._hipcc()
    os.makedirs(OUT, exist_ok=True)
    objs, cmds = [], []
    for src in _b.SOURCES:
        obj = os.path.join(OUT, src.replace(".hip", ".o"))
        objs.append(obj)
        flags = [f if f != "-O3" else "-O1" for f in _b.HIPCC_FLAGS]
        cmds.append([hipcc, *flags, *HOST_SAN, *_b.KERNEL_ONLY_FLAGS.get(src, []), "-c",
                     os.path.join(_b.CSRC, src), "-o", obj])
    with ThreadPoolExecutor(len(cmds)) as ex:
        list(ex.map(_b._run, cmds))
    rocm_lib = "/opt/rocm/lib"
    san_dir = os.path.dirname(subprocess.run([CLANGXX, "-print-file-name=libclang_rt.asan-x86_64.so"],
                                             capture_output=True, text=True).stdout.strip())
    _b._run([CLANGXX, "-shared", "-fPIC", *LINK_SAN, *objs, "-o", LIB, f"-L{rocm_lib}", "-lamdhip64",
             *_b.EXTRA_LIBS, f"-Wl,-rpath,{rocm_lib}", f"-Wl,-rpath,{san_dir}"])
    _b._run([CLANGXX, "-O1", "-g", *LINK_SAN, "-I", os.path.join(_b.ROOT, "include"),
             os.path.join(_b.CSRC, "fa_abi_check.cpp"), "-o", DRIVER, f"-L{OUT}", "-lfa_san",
             f"-Wl,-rpath,{OUT}", f"-Wl,-rpath,{rocm_lib}", f"-Wl,-rpath,{san_dir}"])
    return DRIVER


def run_driver() -> subprocess.CompletedProcess:
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return subprocess.run([DRIVER], env=env, capture_output=True, text=True, timeout=120)
