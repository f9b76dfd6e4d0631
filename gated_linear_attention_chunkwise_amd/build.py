"""Build the HIP library liblizard_attn.so in-tree for gfx950 (hipcc, no JIT).

Every source under csrc/ is compiled to an object with hipcc and linked into
one shared library next to this file.  ``build()`` always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblizard_attn.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 arithmetic instructions stay off: the compiler would otherwise
    # form them from plain float code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; ROCm is required to build liblizard_attn.so")
    return p


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    hipcc = _hipcc()
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [hipcc, *HIP_FLAGS, "-c", src, "-o", obj]
        if src.endswith(".cpp"):
            cmd.insert(1, "-x")
            cmd.insert(2, "hip")
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{out}")
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, sources()))
    tmp = LIB + ".tmp"
    r = subprocess.run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


def asan_runtime() -> str:
    """Path of the toolchain's AddressSanitizer runtime (to preload into a host process)."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.exists(path):
        raise RuntimeError("AddressSanitizer runtime not found in the ROCm toolchain")
    return path


def build_host_sanitized() -> str:
    """A variant of the library whose host code for the C ABI (validation and dispatch,
    lz_api.cpp) is built with AddressSanitizer and UndefinedBehaviorSanitizer, linked with the
    regular kernel objects (device code is not instrumented).  For CPU-side testing only: load it
    into a process that preloads asan_runtime().  Returns the path of the shared library."""
    objdir = os.path.join(ROOT, "_build")
    objs = [os.path.join(objdir, os.path.basename(f) + ".o") for f in sources() if f.endswith(".hip")]
    if not all(os.path.exists(o) for o in objs):
        build()
    sandir = os.path.join(objdir, "san")
    os.makedirs(sandir, exist_ok=True)
    api = os.path.join(CSRC, "lz_api.cpp")
    obj = os.path.join(sandir, "lz_api.o")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    r = subprocess.run([_hipcc(), f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-x", "hip",
                        "-I", os.path.join(ROOT, "include"), *host_san, "-c", api, "-o", obj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitized build of lz_api.cpp failed:\n" + r.stdout + r.stderr)
    lib = os.path.join(sandir, "liblizard_attn_san.so")
    r = subprocess.run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libasan",
                        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        "-o", lib, obj, *objs], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitized link failed:\n" + r.stdout + r.stderr)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
