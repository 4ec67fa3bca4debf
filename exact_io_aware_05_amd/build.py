"""Compile the HIP sources into ``libfa.so`` next to this file (gfx950).

    python -m exact_io_aware_05_amd.build [-v]

Each source is compiled to an object in parallel, then the objects are
linked into one shared library that exports the C interface of
``include/fa.h``.

The library carries the SHA-256 of what it was built from (every file under
``csrc/``, ``include/fa.h`` and the compiler flags), as the string
``FA_SOURCE_HASH=<hex>`` and through ``fa_source_hash()``.  The loader
compares it with the sources on disk, so a library left over from older
sources is rebuilt (or refused) instead of run.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
BUILD_DIR = os.path.join(PKG, "_build")
SOURCES = ("fa_api.hip", "fa_prefill.hip", "fa_splitkv.hip", "fa_backward.hip",
           "fa_prefill_fp8.hip")
# Kernel sources never produce NaN from valid inputs; -fno-honor-nans lets
# fmaxf map to v_max_f32 without canonicalising its operands.  The host
# validation layer (fa_api.hip) must keep NaN semantics for its checks.
# The KV-split kernels run one wave per SIMD, so each may use the 256 AGPRs
# beside its 256 VGPRs: with the matrix-product accumulators kept in VGPRs
# (-amdgpu-mfma-vgpr-form) the register allocator moves its overflow into
# AGPRs (register-to-register copies) instead of spilling to scratch memory,
# which the compiler's default choice does at d = 256.  Measured on MI355X:
# decode at d = 256 11% faster, with a 4096-key window 21% faster.
EXTRA = {"fa_prefill.hip": ["-fno-honor-nans"],
         "fa_splitkv.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "fa_backward.hip": ["-fno-honor-nans"],
         "fa_prefill_fp8.hip": ["-fno-honor-nans"]}
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Wall", "-Wno-unused-function",
        # no packed fp32 (v_pk_*_f32) instructions anywhere
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def source_files():
    """Every input of the build, in a fixed order: the HIP sources and
    headers under csrc/, then the public header."""
    names = sorted(n for n in os.listdir(CSRC) if n.endswith((".hip", ".h")))
    return [os.path.join(CSRC, n) for n in names] + [os.path.join(INCLUDE, "fa.h")]


def source_hash() -> str:
    """SHA-256 over the build's inputs (file names and contents) and the
    compiler flags; the library is stale when its embedded value differs."""
    h = hashlib.sha256()
    for path in source_files():
        h.update(os.path.relpath(path, ROOT).encode() + b"\0")
        with open(path, "rb") as f:
            data = f.read()
        h.update(len(data).to_bytes(8, "little") + data)
    flags = hash_flags(_flags()) + [f"{k}:{' '.join(v)}"
                                    for k, v in sorted(EXTRA.items())]
    h.update("\0".join(flags).encode())
    return h.hexdigest()


def hash_flags(flags):
    """Compiler flags as they enter a hash: paths inside the repository made
    relative to its root, so a copy of the tree elsewhere hashes the same."""
    return [f.replace(ROOT + os.sep, "./") for f in flags]


HASH_MARK = b"FA_SOURCE_HASH="


def embedded_hash(lib_path: str = LIB):
    """The source hash recorded in a built library (read from the file,
    without loading it), or None when it has none."""
    try:
        with open(lib_path, "rb") as f:
            data = f.read()
    except OSError:
        return None
    i = data.find(HASH_MARK)
    if i < 0:
        return None
    hexd = data[i + len(HASH_MARK):i + len(HASH_MARK) + 64]
    try:
        return hexd.decode("ascii") if len(hexd) == 64 and int(hexd, 16) >= 0 else None
    except ValueError:
        return None


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the gfx feature flag; that is harmless
    err = "\n".join(line for line in p.stderr.splitlines()
                    if "not a recognized feature" not in line)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    digest = source_hash()
    objs = []
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        extra = list(EXTRA.get(src, []))
        if src == "fa_api.hip":
            extra.append(f'-DFA_SOURCE_HASH="{digest}"')
        jobs.append([cc, *_flags(), *extra, "-c",
                     os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
         verbose)
    if embedded_hash(tmp) != digest:
        raise RuntimeError("built library does not carry its source hash")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
