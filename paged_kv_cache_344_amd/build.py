"""Build libpa.so in-tree with hipcc for gfx950 (always recompiles), then check its
machine code (codecheck.py).  Each source is compiled on its own, in parallel, and
the objects are linked into one shared library."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libpa.so")
# diagnostic build: the same library with the decode kernel recording per-item timestamps
TRACE_LIB_PATH = os.path.join(PKG, "libpa_trace.so")
SOURCES = ["decode.hip", "cache_write.hip", "copy_blocks.hip", "multi_token.hip", "noalloc.hip",
           "read_probe.hip", "pa_api.cpp", "block_manager.cpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa.so)")


# Device code never uses packed fp32 arithmetic (v_pk_add/mul/fma_f32): the target
# feature below switches it off for the gfx950 pass.  The x86 host pass does not know
# the feature and says so in a warning, which is harmless.  codecheck.py verifies the
# result on the built code objects.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Wno-unused-command-line-argument",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def compile_command(src: str, obj: str, extra=()) -> list:
    return [hipcc(), *FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src),
            "-o", obj]


def link_command(objs: list, out: str) -> list:
    return [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out]


def build(verbose: bool = False, check: bool = True, trace: bool = False) -> str:
    """Build libpa.so (or, with trace, the diagnostic libpa_trace.so whose decode kernel
    records per-item timestamps; see trace_decode.py) and return its path."""
    out_path = TRACE_LIB_PATH if trace else LIB_PATH
    extra = ["-DPA_DECODE_TRACE"] if trace else []
    with tempfile.TemporaryDirectory(prefix="libpa_build_") as tmp:
        objs = [os.path.join(tmp, s + ".o") for s in SOURCES]

        def one(i):
            cmd = compile_command(SOURCES[i], objs[i], extra)
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)

        workers = max(1, min(len(SOURCES), os.cpu_count() or 1))
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, range(len(SOURCES))))
        tmp_lib = os.path.join(tmp, "libpa.so")
        cmd = link_command(objs, tmp_lib)
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        if check:
            from . import codecheck
            rep = codecheck.check(tmp_lib)
            if verbose:
                print(f"machine-code checks passed: {rep}", flush=True)
        shutil.copyfile(tmp_lib, out_path + ".tmp")
        os.chmod(out_path + ".tmp", 0o755)
        os.replace(out_path + ".tmp", out_path)
    return out_path


if __name__ == "__main__":
    import sys
    sys.path.insert(0, ROOT)
    from paged_kv_cache_344_amd import build as _b
    print(_b.build(verbose=True))
