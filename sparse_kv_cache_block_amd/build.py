"""Build libsparsekv.so (gfx950) in-tree: csrc/*.hip with hipcc, and the host
code of the hybrid step (csrc/*.cpp, OpenMP) with the system C++ compiler."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsparsekv.so")
BUILD_DIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         # packed fp32 arithmetic stays off: the compiler must not form v_pk_* fp32 ops
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(HERE, "..", "include")]


CXX = os.environ.get("CXX_HOST", "g++")
# x86-64-v3 (AVX2, FMA, F16C): every MI355X host CPU has it
CXX_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-fopenmp", "-march=x86-64-v3", "-Wall"]

# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build (CPU runs only:
# the device code is not instrumented).  Everything is compiled with clang so
# that one sanitizer runtime (clang's, preloaded) serves the whole process.
SAN_DIR = os.path.join(HERE, "_asan")
SAN_LIB = os.path.join(SAN_DIR, "libsparsekv.so")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined"]
SAN_HIP = [f for flag in SAN for f in ("-Xarch_host", flag)] + ["-Xarch_host", "-fno-omit-frame-pointer",
                                                                "-Xarch_host", "-g"]
SAN_CXX = ["-O1", "-g", "-std=c++17", "-fPIC", "-fopenmp", "-march=x86-64-v3", "-fno-omit-frame-pointer", *SAN]


def sources(src_dir: str = CSRC) -> list[str]:
    return sorted(glob.glob(os.path.join(src_dir, "*.hip")) + glob.glob(os.path.join(src_dir, "*.cpp")))


def build(verbose: bool = False, extra_flags=(), out: str = LIB, build_dir: str = BUILD_DIR,
          src_dir: str = CSRC, sanitize: bool = False) -> str:
    """Compile every HIP source and link the shared library; always rebuilds.
    sanitize=True builds the host-sanitized library into _asan/ instead."""
    if sanitize:
        out, build_dir = SAN_LIB, os.path.join(SAN_DIR, "obj")
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources(src_dir)

    def compile_one(src: str) -> str:
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        if src.endswith(".cpp"):
            cmd = [CLANGXX, *SAN_CXX, "-c", src, "-o", obj] if sanitize else [CXX, *CXX_FLAGS, "-c", src, "-o", obj]
        else:
            cmd = [HIPCC, *FLAGS, *(SAN_HIP if sanitize else ()), *extra_flags, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"{cmd[0]} failed for {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = out + ".tmp"
    # the host code's OpenMP runtime is GCC's (the one the rest of the process uses)
    if sanitize:
        # the sanitizer runtime and LLVM's OpenMP runtime come from the preloaded process
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
               "-L/opt/rocm/llvm/lib", "-lomp", "-Wl,-rpath,/opt/rocm/llvm/lib"]
    else:
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-lgomp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import sys
    print(build(verbose=True, sanitize="--sanitize" in sys.argv))
