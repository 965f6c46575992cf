"""Build ``libpagedattn.so`` for gfx950 with hipcc, in-tree.

``python -m paged_kv_cache_142_amd.build`` compiles every ``csrc/*.hip``
translation unit in parallel and links the shared library next to this file,
and beside it the checked build ``libpagedattn_checked.so``: the same
library with the translation units that hold entry points compiled again
with ``PA_CHECK_CONTENTS=1``, which validates device contents on the host
before each launch (a debugging aid; the kernels are the same objects).
All device code is compiled for gfx950 only, with packed fp32 arithmetic
disabled.
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
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libpagedattn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
CHECKED_LIB_PATH = os.path.join(PKG, "libpagedattn_checked.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libpagedattn")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _has_entry_points(src):
    with open(src) as f:
        return 'extern "C"' in f.read()


def _link(hipcc, objs, out_path):
    tmp = out_path + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, out_path)


def build(extra_flags=(), out_path=LIB_PATH, verbose=False, jobs=None, checked_out_path=None):
    """Compile and link; returns the path of the shared library.  With
    ``checked_out_path``, also links the checked build there."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    flags = COMMON_FLAGS + list(extra_flags)
    srcs = sources()
    checked_srcs = [src for src in srcs if _has_entry_points(src)] if checked_out_path else []

    def compile_one(job):
        src, checked = job
        job_flags = flags + (["-DPA_CHECK_CONTENTS=1"] if checked else [])
        tag = str(abs(hash((tuple(job_flags), out_path))) % 10 ** 8)
        obj = os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + f".{tag}.o")
        cmd = [hipcc, *job_flags, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
        return obj

    jobs_list = [(src, False) for src in srcs] + [(src, True) for src in checked_srcs]
    workers = jobs or max(1, min(len(jobs_list), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(compile_one, jobs_list))
    release = objs[:len(srcs)]
    _link(hipcc, release, out_path)
    if checked_out_path:
        replaced = dict(zip(checked_srcs, objs[len(srcs):]))
        _link(hipcc, [replaced.get(src, obj) for src, obj in zip(srcs, release)], checked_out_path)
    return out_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, checked_out_path=CHECKED_LIB_PATH))
