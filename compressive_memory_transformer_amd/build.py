"""Builds the HIP library libinfini_attn.so in-tree for gfx950.

    python -m compressive_memory_transformer_amd.build [-v] [--sanitize]

Every ``csrc/*.hip`` file is compiled to an object with hipcc (in parallel) and
the objects are linked into ``libinfini_attn.so`` next to this file.

``--sanitize`` builds a second copy whose host code (argument validation,
workspace carving, launch sequences) is instrumented with AddressSanitizer and
UndefinedBehaviorSanitizer, into ``_build/sanitize/libinfini_attn_sanitize.so``.
The device code is compiled as usual (no GPU sanitizer).  It is loaded only by
the CPU check that runs the C-ABI tests under the sanitizers
(``INFINI_ATTN_LIB`` points the binding at it; the sanitizer runtime has to be
preloaded, ``sanitizer_runtime()`` names it).
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_NAME = "libinfini_attn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-variable",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# host-only sanitizers: each -fsanitize applies to the host compilation only
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined", "-g"]
SANITIZE_DIR = os.path.join(BUILD_DIR, "sanitize")
SANITIZE_LIB = os.path.join(SANITIZE_DIR, "libinfini_attn_sanitize.so")


def sanitizer_runtime() -> str:
    """The ASan runtime of the ROCm clang (to preload into a process that loads the
    sanitized library)."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("ASan runtime of the ROCm clang not found")
    return hits[-1]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build the library")
    return path


def _compile(src: str, verbose: bool, sanitize: bool = False) -> str:
    out_dir = SANITIZE_DIR if sanitize else BUILD_DIR
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    flags = [*HIPCC_FLAGS, *SANITIZE_FLAGS] if sanitize else HIPCC_FLAGS
    cmd = [hipcc(), *flags, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    return obj


def build(verbose: bool = False, jobs: int | None = None, sanitize: bool = False) -> str:
    """Compiles every HIP source and links the shared library; returns its path
    (with ``sanitize``, the host-sanitized copy described above)."""
    os.makedirs(SANITIZE_DIR if sanitize else BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not sources:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    jobs = jobs or min(len(sources), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize), sources))
    out = SANITIZE_LIB if sanitize else LIB_PATH
    tmp = out + ".tmp"
    link_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-shared-libsan"] if sanitize else []
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_san, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
