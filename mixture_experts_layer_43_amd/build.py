"""Build libmoe.so (gfx950) in-tree with hipcc.

    python -m mixture_experts_layer_43_amd.build

Each .hip under csrc/ is compiled separately (in parallel) and linked into
mixture_experts_layer_43_amd/libmoe.so.  The checked library
libmoe_debug.so is linked from the same objects except the C-ABI layer,
which is compiled again with MOE_DEBUG (moe_permute then verifies
caller-supplied expert ids before using them), and libmoe_asan.so likewise
with the host side of that layer under AddressSanitizer (for the host tests;
it needs the sanitizer runtime preloaded).  Object files go to _build/ at the
repository root.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
DEBUG_LIB = os.path.join(PKG, "libmoe_debug.so")
# Host-side AddressSanitizer build of the C-ABI layer (argument checks,
# workspace layout); the device code is not instrumented.
ASAN_LIB = os.path.join(PKG, "libmoe_asan.so")
ASAN_HOST = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")
# The C-ABI layer: the one source compiled again for the checked and
# sanitizer builds.
DEBUG_SOURCE = "api.hip"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# Packed fp32 VALU ops are switched off for every device compile.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(job) -> str:
    src, variant = job
    out_dir = os.path.join(BUILD, variant) if variant else BUILD
    obj = os.path.join(out_dir, os.path.basename(src)[:-4] + ".o")
    extra = {"": [], "debug": ["-DMOE_DEBUG"], "asan": ["-g", *ASAN_HOST]}[variant]
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib, extra=()):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    # A kernel whose host stub was not emitted links fine but fails at load.
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in nm.stdout.splitlines() if "device_stub" in l]
    if missing:
        raise RuntimeError("kernel host stubs missing from " + os.path.basename(lib) + ":\n" +
                           "\n".join(missing))
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    for v in ("debug", "asan"):
        os.makedirs(os.path.join(BUILD, v), exist_ok=True)
    srcs = sources()
    api_src = os.path.join(CSRC, DEBUG_SOURCE)
    jobs = [(s, "") for s in srcs] + [(api_src, "debug"), (api_src, "asan")]
    with ThreadPoolExecutor(max(1, min(len(jobs), os.cpu_count() or 1))) as ex:
        objs = list(ex.map(_compile, jobs))
    release, dbg_obj, asan_obj = objs[:-2], objs[-2], objs[-1]
    api_obj = DEBUG_SOURCE[:-4] + ".o"
    swap = lambda o: [o if os.path.basename(r) == api_obj else r for r in release]
    _link(release, LIB)
    _link(swap(dbg_obj), DEBUG_LIB)
    _link(swap(asan_obj), ASAN_LIB, ASAN_HOST[:2])
    if verbose:
        print(f"built {LIB}, {os.path.basename(DEBUG_LIB)} and {os.path.basename(ASAN_LIB)} "
              f"from {len(srcs)} sources", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
