"""Build libmuon.so (gfx950) in place with hipcc, and the binding's argument
marshalling module (_marshal, plain C++ against torch's headers, g++).

    python -m matrix_aware_optimizer_libmuon_amd.build
    python -m matrix_aware_optimizer_libmuon_amd.build --asan OUT_DIR

The second form builds a copy of the library whose host code (argument
checks, workspace planning, descriptor tables, the staging ring) is compiled
with AddressSanitizer; the device code is the same.  Load it by pointing
MUON_LIB at OUT_DIR/libmuon.so, with the sanitizer runtime (asan_runtime())
preloaded into a process that is not itself instrumented, e.g. Python:
    LD_PRELOAD=<asan_runtime()> ASAN_OPTIONS=detect_leaks=0 MUON_LIB=... python ...
"""
from __future__ import annotations

import os
import subprocess
import sys
import sysconfig

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmuon.so")
# (source, extra flags).  The tile-128 GEMM unit keeps its MFMA accumulators
# in ordinary vector registers (they fit at that tile size; the
# accumulator-register form made the compiler copy them inside the K loop).
SOURCES = [
    ("muon_kernels.hip", []),
    ("muon_gemm256.hip", []),
    ("muon_gemm128.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]),
    ("muon_fused.hip", []),
    ("muon_noalloc.hip", []),
    ("muon_api.cpp", []),
]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


MARSHAL = os.path.join(PKG, "_marshal" + sysconfig.get_config_var("EXT_SUFFIX"))


def _start(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def _finish(job, verbose):
    cmd, proc = job
    out, _ = proc.communicate()
    out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"{os.path.basename(cmd[0])} failed ({proc.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)


def _run(cmd, verbose):
    _finish(_start(cmd, verbose), verbose)


def _marshal_cmd(out):
    from torch.utils import cpp_extension as ce
    import torch
    abi = int(torch._C._GLIBCXX_USE_CXX11_ABI)
    libdir = ce.library_paths()[0]
    return ["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-Wall",
            f"-D_GLIBCXX_USE_CXX11_ABI={abi}", "-DTORCH_EXTENSION_NAME=_marshal",
            "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
            *[f"-I{p}" for p in ce.include_paths()], f"-I{sysconfig.get_paths()['include']}",
            os.path.join(CSRC, "marshal.cpp"), "-o", out,
            f"-L{libdir}", "-lc10", "-ltorch", "-ltorch_cpu", "-ltorch_python", f"-Wl,-rpath,{libdir}"]


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel), link libmuon.so next to this file
    and build the marshalling module; returns the library's path."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs, objs = [], []
    for src, extra in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        jobs.append(_start([HIPCC, *FLAGS, *extra, "-c", "-o", obj, os.path.join(CSRC, src)], verbose))
        objs.append(obj)
    marshal_tmp = MARSHAL + ".tmp"
    jobs.append(_start(_marshal_cmd(marshal_tmp), verbose))
    try:
        for job in jobs:
            _finish(job, verbose)
    finally:
        for _, proc in jobs:
            if proc.poll() is None:
                proc.kill()
                proc.wait()
    os.replace(marshal_tmp, MARSHAL)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


def asan_runtime() -> str | None:
    """Path of the clang AddressSanitizer runtime of the ROCm toolchain."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_asan(out_dir: str, verbose: bool = False) -> str:
    """libmuon.so in out_dir with the host dispatcher under AddressSanitizer
    (hipcc: -Xarch_host before the sanitizer flag keeps it off the device
    code).  The kernel objects are compiled as usual."""
    os.makedirs(out_dir, exist_ok=True)
    jobs, objs = [], []
    for src, extra in SOURCES:
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        if src == "muon_api.cpp":
            extra = [*extra, "-Xarch_host", "-fsanitize=address", "-fno-omit-frame-pointer", "-g"]
        jobs.append(_start([HIPCC, *FLAGS, *extra, "-c", "-o", obj, os.path.join(CSRC, src)], verbose))
        objs.append(obj)
    try:
        for job in jobs:
            _finish(job, verbose)
    finally:
        for _, proc in jobs:
            if proc.poll() is None:
                proc.kill()
                proc.wait()
    out = os.path.join(out_dir, "libmuon.so")
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libasan",
          "-Xarch_host", "-fsanitize=address", "-o", out, *objs], verbose)
    return out


if __name__ == "__main__":
    if "--asan" in sys.argv:
        print(build_asan(sys.argv[sys.argv.index("--asan") + 1], verbose="-q" not in sys.argv))
    else:
        print(build(verbose="-q" not in sys.argv))
