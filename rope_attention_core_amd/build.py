"""Build libsa3attn.so in-tree with hipcc for gfx950.

    python -m rope_attention_core_amd.build [--asm DIR]
    python -m rope_attention_core_amd.build --host-sanitize DIR

--host-sanitize builds a second copy of the library into DIR whose host code (the
C-ABI layer and the RoPE table: argument validation, stride, extent and overlap
arithmetic) is compiled by g++ with AddressSanitizer and UndefinedBehaviorSanitizer;
the kernels are the in-tree objects, unchanged. The binding loads it when the
environment variable SA3ATTN_LIB names it; run Python with the sanitizer runtime
preloaded:

    SA3ATTN_LIB=DIR/libsa3attn.so LD_PRELOAD=$(gcc -print-file-name=libasan.so) \
    ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \
    python -m pytest tests/test_abi.py -m "not gpu"

The library is one shared object: the C-ABI layer (csrc/api.cpp), the host RoPE
table (csrc/rope_table.cpp) and the kernels (csrc/attn_fwd.hip for full attention and
wide windows, csrc/attn_prep.hip its optional pre-pass, csrc/attn_narrow.hip for
windows of half-width <= 32 and short sequences). It is written next to this file so
that it travels with the source tree.
"""

import argparse
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libsa3attn.so")

ARCH = "gfx950"
SOURCES = ["attn_fwd.hip", "attn_narrow.hip", "attn_prep.hip", "attn_split.hip", "scratch.hip", "api.cpp",
           "rope_table.cpp"]
# Packed FP32 instructions are kept out of the device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"build failed ({res.returncode}):\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose=False, asm_dir=None):
    """Compile every source (in parallel, one process each) and link libsa3attn.so
    (always rebuilds)."""
    from concurrent.futures import ThreadPoolExecutor

    cc = hipcc()
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs, objs = [], []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(objdir, src + ".o")
        cmd = [cc, f"--offload-arch={ARCH}", *COMMON]
        if src.endswith(".hip"):
            cmd += ["-x", "hip", *DEVICE_FLAGS]
        jobs.append(cmd + ["-c", path, "-o", obj])
        objs.append(obj)
        if asm_dir and src.endswith(".hip"):
            os.makedirs(asm_dir, exist_ok=True)
            jobs.append([cc, f"--offload-arch={ARCH}", *COMMON, "-x", "hip", *DEVICE_FLAGS, "--cuda-device-only",
                         "-S", path, "-o", os.path.join(asm_dir, src + ".s")])
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        for f in [pool.submit(_run, cmd, verbose) for cmd in jobs]:
            f.result()
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


HOST_SOURCES = ["api.cpp", "rope_table.cpp"]


def build_host_sanitized(out_dir, verbose=False):
    """The library with its host sources built by g++ under ASan + UBSan (see the module
    docstring); the kernel objects come from an in-tree build()."""
    build(verbose=verbose)
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    gxx = shutil.which("g++") or "g++"
    rocm_inc = os.path.join(os.path.dirname(os.path.dirname(hipcc())), "include")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(out_dir, src + ".san.o")
        cmd = [gxx, "-O1", "-g", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{rocm_inc}",
               f"-I{INCLUDE}", f"-I{CSRC}", *san, "-c", os.path.join(CSRC, src), "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    kernels = [os.path.join(objdir, src + ".o") for src in SOURCES if src.endswith(".hip")]
    lib = os.path.join(out_dir, "libsa3attn.so")
    rocm_lib = os.path.join(os.path.dirname(rocm_inc), "lib")
    _run([gxx, "-shared", *san, *objs, *kernels, f"-L{rocm_lib}", f"-Wl,-rpath,{rocm_lib}", "-lamdhip64",
          "-o", lib], verbose)
    return lib


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="also write device assembly into this directory")
    ap.add_argument("--host-sanitize", default=None, metavar="DIR",
                    help="build a copy with ASan/UBSan host code into DIR instead")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    if a.host_sanitize:
        print(build_host_sanitized(a.host_sanitize, verbose=a.verbose))
        return
    print(build(verbose=a.verbose, asm_dir=a.asm))


if __name__ == "__main__":
    sys.exit(main())
