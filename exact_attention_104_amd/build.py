"""Builds libfa_mi355x.so, the gfx950 HIP library, in the package directory.

Each ``csrc/*.hip`` file is compiled by hipcc for gfx950 only, then linked into
one shared library that exports the C ABI of ``include/fa.h``. Run
``python -m exact_attention_104_amd.build`` (or ``__graft_entry__.build()``).

``build(sanitize=True)`` (``python -m exact_attention_104_amd.build --host-sanitize``)
builds ``libfa_mi355x_hostsan.so`` instead: the same sources with the host
code (argument validation, dispatch) instrumented by AddressSanitizer and
UndefinedBehaviorSanitizer; the device code is built as usual. It is for CPU
runs of the C-ABI tests only (load it with the sanitizer runtime preloaded,
see ``HOSTSAN_RUNTIME``).
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "libfa_mi355x.so"
HOSTSAN_LIB_NAME = "libfa_mi355x_hostsan.so"
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no NaN inputs are assumed (NaN propagation is outside the contract), which
    # lets fmaxf compile to a single v_max without operand canonicalisation
    "-fno-honor-nans",
    "-I" + os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function",
]


# per-file additions: the d = 256 backward is built with every MFMA in its VGPR
# form (its dK/dV kernel then keeps S and dP out of AGPRs; the flag acts on a
# whole file and slowed the d = 128 instances, hence a file of its own)
FILE_FLAGS = {"fa_bwd_d256.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

# host-only sanitizers: each -fsanitize= applies to the host compilation only
HOSTSAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def hostsan_runtime() -> str | None:
    """The AddressSanitizer runtime of the ROCm clang (to preload), or None."""
    cands = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return cands[-1] if cands else None


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + (".hostsan.o" if sanitize else ".o"))
    extra = FILE_FLAGS.get(os.path.basename(src), [])
    cmd = [HIPCC] + FLAGS + extra + (HOSTSAN_FLAGS if sanitize else []) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = True, sanitize: bool = False) -> str:
    """Compile every HIP source and link the library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), sources))
    out = os.path.join(PKG, HOSTSAN_LIB_NAME if sanitize else LIB_NAME)
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    shutil.move(tmp, out)
    if verbose:
        print("built", out, file=sys.stderr)
    return out


if __name__ == "__main__":
    build(sanitize="--host-sanitize" in sys.argv[1:])
