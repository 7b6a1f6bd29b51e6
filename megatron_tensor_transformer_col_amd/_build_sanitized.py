"""Build libtpcol_san.so: libtpcol with its host code under AddressSanitizer
and UndefinedBehaviorSanitizer (device code as in the release build), for
the CPU-side ABI tests.

    python -m megatron_tensor_transformer_col_amd._build_sanitized

The sanitizers apply to the host side only (each flag after -Xarch_host);
every undefined-behaviour finding aborts.  A process that loads the library
needs the ASan runtime first in line: LD_PRELOAD=asan_runtime().
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import sys

from . import _build

BUILD = os.path.join(_build.ROOT, "_build_san")
LIB = os.path.join(BUILD, "libtpcol_san.so")

SAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]


def asan_runtime() -> str:
    """Path of the clang ASan runtime that matches hipcc's compiler."""
    hip = os.path.dirname(os.path.dirname(os.path.realpath(_build._hipcc())))
    for root in (hip, "/opt/rocm"):
        hits = sorted(glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                             "libclang_rt.asan-x86_64.so")))
        if hits:
            return hits[-1]
    raise RuntimeError("libclang_rt.asan-x86_64.so not found next to hipcc")


def build() -> str:
    hipcc = _build._hipcc()
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(f for f in os.listdir(_build.CSRC) if f.endswith(".hip"))
    objs, jobs = [], []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        for src in sources:
            obj = os.path.join(BUILD, src[:-4] + ".o")
            objs.append(obj)
            cmd = [hipcc, *_build.HIPCC_FLAGS, *_build.EXTRA_FLAGS.get(src, []), *SAN_FLAGS, "-c",
                   os.path.join(_build.CSRC, src), "-o", obj]
            jobs.append(ex.submit(_build._run, cmd))
        for j in jobs:
            j.result()
    tmp = LIB + ".tmp"
    _build._run([hipcc, f"--offload-arch={_build.ARCH}", "-shared", "-fPIC", *SAN_FLAGS, "-shared-libasan",
                 "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
