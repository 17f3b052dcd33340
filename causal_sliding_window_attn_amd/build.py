"""Build libswattn.so in-tree with hipcc for gfx950 (no torch involvement)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libswattn.so")
SOURCES = ["api.cpp", "fwd.hip", "bwd.hip", "decode.hip", "norm.hip"]
HEADERS = ["common.h", "launch.h"]
# measurement helper used by bench.py only (streaming-read reference for the decode roofline)
PROBE_LIB = os.path.join(PKG, "libswattn_probe.so")
PROBE_SOURCES = ["stream_probe.hip"]
ARCH = "gfx950"

# Packed-fp32 VALU forms are switched off for all device code; hipcc's host pass warns that it
# does not know the feature, which is harmless.
HIPFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build libswattn.so")
    return exe


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, src.replace(".", "_") + ".o")
    cmd = [hipcc(), *HIPFLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise and os.environ.get("SWATTN_BUILD_VERBOSE"):
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(extra: list[str] | None = None) -> str:
    """Compile every source for gfx950 and link libswattn.so (and the bench's streaming-read probe
    library) next to this file.  Returns the path of libswattn.so."""
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra or [])
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, extra), srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    return LIB


# Host-side AddressSanitizer build of the library, for the CPU tests of the C ABI (argument
# validation, error text): api.cpp's host code is instrumented (-Xarch_host puts the sanitizer on
# the host compilation only; device code is built as usual), and the result is a separate file.
ASAN_LIB = os.path.join(PKG, "libswattn_asan.so")


def asan_runtime() -> str:
    """Path of the clang ASan runtime that a process loading ASAN_LIB must preload."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the clang AddressSanitizer runtime was not found")
    return path


def build_asan() -> str:
    os.makedirs(BUILD, exist_ok=True)
    asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    def one(src):
        if src != "api.cpp":
            return _compile(src, [])
        obj = _compile(src, asan)
        tagged = obj[:-2] + "_asan.o"
        os.replace(obj, tagged)
        return tagged

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = ASAN_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host",
           "-fsanitize=address", "-shared-libasan", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


if __name__ == "__main__":
    if sys.argv[1:2] == ["--asan"]:
        print(build_asan())
    else:
        print(build(sys.argv[1:]))
