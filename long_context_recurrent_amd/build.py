"""Build libarmt.so (HIP, gfx950) in-tree.

    python -m long_context_recurrent_amd.build        # or build_library()
    python -m long_context_recurrent_amd.build --host-sanitize   # ASan/UBSan host build

Each .hip source under csrc/ is compiled with hipcc for gfx950 into an object
under long_context_recurrent_amd/_build/, then linked into
long_context_recurrent_amd/libarmt.so.  Packed fp32 instructions are disabled
for all device code.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libarmt.so")
ARCH = "gfx950"

DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-function", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libarmt.so)")


def sources() -> list:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Per-source extra device flags.  Attention keeps its MFMA results in
# ordinary VGPRs: the softmax works on every score and accumulator element
# between products, which would otherwise cost a register move each way.
EXTRA: dict = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
               # the memory read unrolls its chunk loops completely (24 chunks at d = 3072)
               "memory_mfma.hip": ["-mllvm", "-pragma-unroll-threshold=200000"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        msg = "\n".join(l for l in proc.stderr.splitlines() if "packed-fp32-ops" not in l)
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{msg}")
    return obj


def build_library(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every HIP source and link libarmt.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{proc.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


# Host sanitizers for the runtime (argument checks, layouts, the scheduler,
# graph bookkeeping): AddressSanitizer and UndefinedBehaviorSanitizer on the
# host code of armt_runtime.hip only -- each flag behind -Xarch_host, so no
# device code is built with them.  The other objects are the regular ones.
SANITIZE = ["-O1", "-g", "-fno-omit-frame-pointer"] + [
    f for opt in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined")
    for f in ("-Xarch_host", opt)]
SAN_LIB = os.path.join(BUILD, "sanitize", "libarmt.so")


def asan_runtime() -> str:
    """Shared AddressSanitizer runtime of the compiler (to preload into a
    process that is not built with it, such as python)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = shutil.which("clang") or "clang"
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return out.stdout.strip()


def build_host_sanitized(verbose: bool = False) -> str:
    """libarmt.so with ASan + UBSan in the host code of the runtime, under
    _build/sanitize/; load it with ARMT_LIBRARY=<path> and the runtime from
    asan_runtime() preloaded."""
    srcs = sources()
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    if not all(os.path.exists(o) for o in objs):
        build_library()
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    rt_src = os.path.join(CSRC, "armt_runtime.hip")
    rt_obj = os.path.join(os.path.dirname(SAN_LIB), "armt_runtime.o")
    flags = [f for f in COMMON if f != "-O3"]
    cmd = [hipcc(), *flags, *DEVICE_FLAGS, *SANITIZE, "-c", rt_src, "-o", rt_obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{proc.stderr}")
    objs = [rt_obj if o.endswith("armt_runtime.o") else o for o in objs]
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-o", SAN_LIB, *objs]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{proc.stderr}")
    if verbose:
        print(f"built {SAN_LIB} (host ASan + UBSan in the runtime)")
    return SAN_LIB


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--host-sanitize":
        build_host_sanitized(verbose=True)
    else:
        build_library(verbose=True)
    sys.exit(0)
