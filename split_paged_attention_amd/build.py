"""Build libspa.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run as a script or through build(); the library lands next to this file
(in-tree), which is where the Python binding loads it from."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libspa.so")
OBJDIR = os.path.join(HERE, "_build")
# The diagnostics build: the same sources with SPA_TIMELINE defined (per-wave
# timeline of the decode producer, include/spa_timeline.h).
TIMELINE_LIB = os.path.join(HERE, "libspa_timeline.so")
TIMELINE_OBJDIR = os.path.join(HERE, "_build_timeline")
SOURCES = ["metadata.hip", "decode_attention.hip", "verify_attention.hip", "api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU forms are kept out of the generated code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC] + DEVICE_FLAGS


def _compile(src: str, verbose: bool, objdir: str = OBJDIR, defines=()) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + [f"-D{d}" for d in defines] + ["-x", "hip", "-c",
                                                            os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)
    return obj


def _build(lib: str, objdir: str, defines, verbose: bool) -> str:
    os.makedirs(objdir, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, objdir, defines), SOURCES))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = True) -> str:
    """libspa.so, the library."""
    return _build(LIB, OBJDIR, (), verbose)


def build_timeline(verbose: bool = True) -> str:
    """libspa_timeline.so, the diagnostics build (not used by the library)."""
    return _build(TIMELINE_LIB, TIMELINE_OBJDIR, ("SPA_TIMELINE",), verbose)


if __name__ == "__main__":
    build()
    if "--timeline" in sys.argv[1:]:
        build_timeline()
    sys.exit(0)
