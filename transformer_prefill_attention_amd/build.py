"""Build ``libpfa.so`` in-tree with hipcc for gfx950.

Every HIP source under ``csrc/`` is compiled and linked into one shared library
next to this file; ``include/`` at the repository root holds the public header.
Packed FP32 instructions are disabled for all device code.

``python build.py --sanitize DIR`` builds a second copy, ``DIR/libpfa_san.so``, whose
host code (argument checks, sequence tables, schedules, workspace layouts, the plan
report) carries AddressSanitizer and UndefinedBehaviorSanitizer instrumentation; the
device code is built as usual.  An executable linked with the sanitizer runtimes loads
it (the test suite's sanitizer drivers do).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpfa.so")
OBJ_DIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result", "-ffp-contract=fast-honor-pragmas"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# host-only instrumentation: every sanitizer flag goes to the host pass alone
SAN_FLAGS = ["-g", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all"]


def _compile(src: str, obj_dir: str = OBJ_DIR, extra=()) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    # the host pass does not know the gfx feature flag; everything else is shown
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if msg.strip():
        sys.stderr.write(msg + "\n")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every ``csrc/*.hip`` and link ``libpfa.so`` (always rebuilds)."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_sanitized(out_dir: str, verbose: bool = True) -> str:
    """``out_dir/libpfa_san.so``: the library with host-side ASan + UBSan (see above)."""
    obj_dir = os.path.join(out_dir, "obj")
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir, SAN_FLAGS), srcs))
    lib = os.path.join(out_dir, "libpfa_san.so")
    subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", lib, *objs],
                   check=True)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "--sanitize":
        build_sanitized(sys.argv[2])
    else:
        build()
