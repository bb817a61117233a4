"""Build libfa.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Run ``python -m exact_attention_forward_fa_amd.build`` (or call ``build()``).
Each source is compiled to an object under ``_build/`` in parallel, then
linked into ``exact_attention_forward_fa_amd/libfa.so``; two debug variants are
built beside it (see POISON_OUT and SANITIZE_OUT).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libfa.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["prefill.hip", "decode.hip", "combine.hip", "append.hip", "backward.hip", "fa_api.cpp"]
ARCH = "gfx950"

# Packed fp32 VALU instructions are turned off for all device code.  IEEE NaN
# semantics stay on: some buffers may hold NaN by contract (the decode workspace,
# cache rows past a sequence's length) and the kernels rely on skipping them.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def _compile(src: str, prefix: str = "", extra=()) -> str:
    obj = os.path.join(BUILD_DIR, prefix + os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
           "-Wno-unused-function", "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + DEVICE_FLAGS + list(extra)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


# Debug builds (both built by build()):
#  * POISON_OUT: the kernels that stage K/V tiles in LDS (prefill, decode) fill
#    those tiles with NaN before first use (FA_LDS_POISON), so a read that a
#    missing barrier lets run ahead of the tile's store turns into NaN in out;
#  * SANITIZE_OUT (CPU only, not shipped): the host layer fa_api.cpp with
#    AddressSanitizer and UndefinedBehaviorSanitizer on its host code, linked with
#    the ordinary kernel objects; the ABI tests load it with the clang ASan
#    runtime preloaded.
POISON_OUT = os.path.join(PKG, "libfa_lds_poison.so")
POISON_SOURCES = ["prefill.hip", "decode.hip"]
SANITIZE_OUT = os.path.join(BUILD_DIR, "sanitize", "libfa_sanitize.so")
HOST_SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime matching hipcc (for LD_PRELOAD)."""
    r = subprocess.run([os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang"),
                        "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.exists(path):
        import glob
        hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
        path = hits[-1] if hits else ""
    return path


def _link(objs, out, extra=()):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp] + list(objs)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {out} failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(os.path.join(BUILD_DIR, "sanitize"), exist_ok=True)
    jobs = [(src, "", []) for src in SOURCES]
    jobs += [(src, "poison_", ["-DFA_LDS_POISON=1"]) for src in POISON_SOURCES]
    jobs += [("fa_api.cpp", "sanitize/", ["-g"] + HOST_SANITIZE_FLAGS)]
    with ThreadPoolExecutor(max_workers=min(6, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    plain = objs[:len(SOURCES)]
    _link(plain, OUT)
    poison = {src: o for (src, pre, _), o in zip(jobs, objs) if pre == "poison_"}
    _link([poison.get(src, o) for src, o in zip(SOURCES, plain)], POISON_OUT)
    san = objs[-1]
    _link([san if src == "fa_api.cpp" else o for src, o in zip(SOURCES, plain)], SANITIZE_OUT,
          extra=["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"])
    if verbose:
        print(f"built {OUT}, {POISON_OUT} and {SANITIZE_OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
