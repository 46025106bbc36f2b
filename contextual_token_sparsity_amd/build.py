"""Builds liblemo.so (all HIP sources, gfx950) in-tree with hipcc.

    python -m contextual_token_sparsity_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "liblemo.so")
SOURCES = ["abi.hip", "block_scores.hip", "predict.hip", "token.hip", "select.hip", "movement.hip", "fused.hip",
           "mlp.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
    # packed fp32 VALU forms are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile every source to an object, then link the shared library
    atomically (a running process that has the old library mapped keeps it)."""
    cc = hipcc()
    objs = []
    with tempfile.TemporaryDirectory(prefix="lemo_build_") as tmp:
        procs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [cc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        errors = []
        for src, p in procs:
            out, _ = p.communicate()
            noise = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
            if p.returncode != 0:
                errors.append(f"{src}:\n" + "\n".join(noise))
            elif verbose and noise:
                print("\n".join(noise))
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
        tmp_lib = LIB + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
        os.replace(tmp_lib, LIB)
    return LIB


HOSTCHECK_LIB = os.path.join(PKG, "liblemo_hostcheck.so")
LLVM_BIN = "/opt/rocm/llvm/bin"


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime that the host-check library needs
    preloaded into a process that was not built with it (python)."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang ASan runtime not found")
    return hits[-1]


def build_host_check(verbose: bool = False) -> str:
    """Every source with its host side (argument validation, launch set-up)
    compiled with AddressSanitizer and UndefinedBehaviorSanitizer (the device
    code is built as usual; sanitizer flags apply to the host pass only), as
    liblemo_hostcheck.so.  The C-ABI tests run against it on the CPU, where
    no kernel is launched, to catch memory errors and undefined behaviour in
    the validation layer."""
    cc = hipcc()
    # host pass only: every sanitizer flag goes right after -Xarch_host
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    objs = []
    with tempfile.TemporaryDirectory(prefix="lemo_hostcheck_") as tmp:
        procs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [cc, *HIPCC_FLAGS, "-g", "-Xarch_host", "-fno-omit-frame-pointer", *san, "-c",
                   os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        errors = []
        for src, p in procs:
            out, _ = p.communicate()
            if p.returncode != 0:
                errors.append(f"{src}:\n" + "\n".join(ln for ln in out.splitlines() if "packed-fp32-ops" not in ln))
        if errors:
            raise RuntimeError("host-check compile failed:\n" + "\n".join(errors))
        tmp_lib = HOSTCHECK_LIB + ".tmp"
        link = [os.path.join(LLVM_BIN, "clang++"), "-shared", "-fPIC", "-shared-libasan"]
        link += ["-fsanitize=address,undefined", "-o", tmp_lib, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                 "-Wl,-rpath,/opt/rocm/lib"]
        r = subprocess.run(link, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("host-check link failed:\n" + r.stdout + r.stderr)
        os.replace(tmp_lib, HOSTCHECK_LIB)
    return HOSTCHECK_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    if "--host-check" in sys.argv:
        print(build_host_check(verbose="-v" in sys.argv))
