"""Build libprope.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: python -m position_remapped_rope_amd.build [-v] [--sanitize OUT.so | --trace OUT.so]

--sanitize builds a copy whose host code (argument checks, launch set-up,
integer helpers) carries AddressSanitizer and UndefinedBehaviorSanitizer; the
device code is built as usual. Load it with the ASan runtime preloaded
(libclang_rt.asan-x86_64.so), for CPU-side tests.

--trace builds a copy whose bf16 prefill kernel records item-phase timestamps
(PROPE_ITEM_TRACE=1) and exports prope_item_trace_read; `bench.py --only LEG
--item-trace` run with PROPE_LIB_PATH=OUT.so summarises them. Not for
production use: the timestamps cost a few instructions per item.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libprope.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "rope_apply.hip", "prefill_bf16.hip", "prefill_fp32.hip", "decode_bf16.hip", "decode_scratch.hip",
           "bifocal_unfused.hip"]

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


# host-only sanitizers: every -fsanitize= is bound to the host pass
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """The clang ASan runtime that a process loading a sanitized build must preload."""
    import glob
    cands = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not cands:
        raise RuntimeError("clang ASan runtime not found")
    return cands[-1]


def _compile(src: str, verbose: bool, build_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    # device sources: no kernel relies on NaN semantics, so max() needs no
    # canonicalisation; host argument checks (api.cpp) keep IEEE NaN handling
    lang = ["-x", "hip", "-fno-honor-nans"] if src.endswith(".hip") else []
    cmd = [_hipcc(), *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


TRACE_FLAGS = ["-DPROPE_ITEM_TRACE=1"]


def build(verbose: bool = False, sanitize_out: str = "", trace_out: str = "") -> str:
    """Compile every source (in parallel) and link libprope.so; returns its path.
    With sanitize_out, link a host-sanitized copy there instead; with
    trace_out, a copy with item-phase tracing."""
    if sanitize_out and trace_out:
        raise ValueError("choose one of sanitize_out and trace_out")
    build_dir = os.path.join(BUILD_DIR, "asan") if sanitize_out else \
        os.path.join(BUILD_DIR, "trace") if trace_out else BUILD_DIR
    extra = SANITIZE_FLAGS if sanitize_out else TRACE_FLAGS if trace_out else []
    out = sanitize_out or trace_out or OUT
    os.makedirs(build_dir, exist_ok=True)
    os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, extra), SOURCES))
    tmp = out + ".tmp"
    cmd = [_hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", *extra, "-shared-libsan", "-o", tmp, *objs] \
        if sanitize_out else [_hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    san = sys.argv[sys.argv.index("--sanitize") + 1] if "--sanitize" in sys.argv else ""
    tr = sys.argv[sys.argv.index("--trace") + 1] if "--trace" in sys.argv else ""
    print(build(verbose="-v" in sys.argv, sanitize_out=san, trace_out=tr))
