"""Build libdcp.so (HIP, gfx950) in-tree with hipcc.

Usage: ``python -m sequence_sharded_paged_amd.build`` (or ``build()``).
Every HIP source is compiled for gfx950 only, with packed-fp32 instructions
disabled, then linked into ``sequence_sharded_paged_amd/lib/libdcp.so``.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(HERE, "lib")
OBJDIR = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(LIBDIR, "libdcp.so")

SOURCES = ["abi.cpp", "layout.hip", "merge.hip", "attn_generic.hip", "attn_gqa.hip", "attn_mla.hip", "kv_write.hip", "gather.hip", "probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer (the device code is
# built as usual): for the CPU-only checks of the C ABI's host paths.
SANITIZE_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                  "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer").split()
SANITIZED_LIB = os.path.join(ROOT, "_build", "sanitized", "libdcp.so")


def _compile(src: str, objdir: str = OBJDIR, extra=()) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Build libdcp.so; with ``sanitize`` the host code is instrumented and the
    library goes to ``_build/sanitized/`` (load it with the ASan runtime
    preloaded)."""
    objdir = os.path.join(ROOT, "_build", "obj_sanitized") if sanitize else OBJDIR
    lib = SANITIZED_LIB if sanitize else LIB
    extra = SANITIZE_FLAGS if sanitize else ()
    os.makedirs(objdir, exist_ok=True)
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, objdir, extra), SOURCES))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
