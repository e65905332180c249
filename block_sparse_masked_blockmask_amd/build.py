"""Build the HIP library libflexattn.so in-tree for gfx950.

Compiles every source under csrc/ with hipcc into one shared object next to this file.
All HIP code is built with packed-fp32 instructions disabled (they are avoided on this
hardware; hipcc's host pass warns that it does not know the feature, which is harmless).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libflexattn.so")
SOURCES = ["api.cpp", "blockmask.hip", "fwd.hip", "fwd_dense.hip", "fwd_pipe.hip", "quant.hip", "bwd.hip", "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-I" + INCLUDE, "-I" + CSRC,
]


def build(verbose: bool = False) -> str:
    """Compile all sources (always) and link libflexattn.so; returns its path."""
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, cmd, pr in procs:
        out, _ = pr.communicate()
        text = out.decode(errors="replace")
        if pr.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text)
    if failed:
        msg = "\n".join(f"--- {s} ---\n{t}" for s, t in failed)
        raise RuntimeError("HIP build failed:\n" + msg)
    tmp = LIB + ".tmp"
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, LIB)
    return LIB


# Host sources of the C-ABI layer (argument validation, the host BlockMask builder, the
# allocation-free entry point's bookkeeping): the part a sanitized build instruments.
HOST_SOURCES = ["api.cpp", "noalloc.hip"]
SANITIZED_LIB = os.path.join(ROOT, "_build", "sanitized", "libflexattn_sanitized.so")


def build_sanitized() -> str:
    """Build the C-ABI layer with AddressSanitizer and UndefinedBehaviorSanitizer on its host code
    only (-Xarch_host: the GPU code is not instrumented), linked against the regular library for
    the kernel launchers. For the CPU tests of the host logic; load it with the sanitizer runtime
    preloaded (sanitizer_runtime()) and FLEXATTN_LIBRARY pointing at it. Returns its path."""
    if not os.path.exists(LIB):
        build()
    outdir = os.path.dirname(SANITIZED_LIB)
    os.makedirs(outdir, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(outdir, src + ".o")
        cmd = [HIPCC, *[f for f in FLAGS if f != "-O3"], "-O1", *san, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        if r.returncode != 0:
            raise RuntimeError(f"sanitized build of {src} failed:\n" + r.stdout.decode(errors="replace"))
        objs.append(obj)
    tmp = SANITIZED_LIB + ".tmp"
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *san, "-shared-libasan", "-o", tmp, *objs,
            "-L" + HERE, "-l:libflexattn.so", "-Wl,-rpath," + HERE]
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("sanitized link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, SANITIZED_LIB)
    return SANITIZED_LIB


def sanitizer_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (to preload into the test process)."""
    out = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE,
                         stderr=subprocess.DEVNULL).stdout.decode().strip()
    if not out or not os.path.isabs(out) or not os.path.exists(out):
        import glob
        cands = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        out = cands[0] if cands else ""
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
