"""Build libwkv.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m linear_recurrent_attention_amd.build [--asm DIR]

hipcc cross-compiles without a GPU.  Every translation unit is compiled with
packed-FP32 instructions disabled (``-target-feature -packed-fp32-ops``); only
the ``WKV_API`` symbols are exported.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libwkv.so")
SOURCES = ["wkv_api.hip", "wkv_forward.hip", "wkv_lookback.hip", "wkv_step.hip",
           "wkv_backward.hip", "wkv_shift.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument",
            "-Wfloat-conversion"]


def build(asm_dir: str | None = None, verbose: bool = False) -> str:
    objdir = os.path.abspath(asm_dir) if asm_dir else os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if asm_dir:
            cmd += ["-save-temps=obj"]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True, cwd=objdir)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libwkv.so failed")
    os.replace(tmp, LIB)
    return LIB


SAN_DIR = os.path.join(PKG, "_build", "san")
SAN_LIB = os.path.join(SAN_DIR, "libwkv_san.so")


def build_sanitized(verbose: bool = False) -> str:
    """A copy of the library for host-side checks on a machine without a GPU:
    the host code (argument checks, size arithmetic, caches) built with
    AddressSanitizer and UndefinedBehaviorSanitizer, every finding fatal; the
    device code is built without optimisation (it never runs from this copy)
    and without sanitizers.  Load it with the sanitizer runtime preloaded."""
    os.makedirs(SAN_DIR, exist_ok=True)
    cc = hipcc()
    flags = [f"--offload-arch={ARCH}", "-O1", "-Xarch_device", "-O0", "-std=c++17", "-fPIC",
             "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument",
             "-Xarch_host", "-g", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all"]

    def compile_one(src):
        obj = os.path.join(SAN_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True, cwd=SAN_DIR)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc (sanitized host) failed on {src}")
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libasan", "-o", SAN_LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of the sanitized library failed")
    return SAN_LIB


def sanitizer_runtime() -> str | None:
    """The AddressSanitizer runtime of the compiler that built SAN_LIB."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    for cand in (clang, "/opt/rocm/llvm/bin/clang"):
        if not os.path.exists(cand):
            continue
        r = subprocess.run([cand, "-print-runtime-dir"], capture_output=True, text=True)
        if r.returncode != 0:
            continue
        rt = r.stdout.strip()
        # per-target layout first, then the older lib/linux one beside it
        for d, name in ((rt, "libclang_rt.asan.so"),
                        (os.path.join(os.path.dirname(rt), "linux"),
                         "libclang_rt.asan-x86_64.so")):
            p = os.path.join(d, name)
            if os.path.exists(p):
                return p
    return None


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="keep -save-temps output (ISA) in this folder")
    ap.add_argument("--sanitized", action="store_true",
                    help="build the host-sanitized copy for CPU-only checks instead")
    ap.add_argument("-v", action="store_true")
    args = ap.parse_args()
    print(build_sanitized(args.v) if args.sanitized else build(args.asm, args.v))
