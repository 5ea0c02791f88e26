"""Build libgdnq.so in-tree with hipcc for gfx950.

Each source is compiled to an object in parallel, then linked.  Flags:
  * -ffp-contract=off: no implicit fused multiply-add, so the codec's
    operations round one at a time; kernels ask for fmaf() explicitly;
  * -fhip-fp32-correctly-rounded-divide-sqrt: IEEE division and sqrt;
  * -fno-gpu-flush-denormals-to-zero: fp32 subnormals are kept;
  * -mno-amdgpu-ieee -fno-honor-nans: NaN inputs are unsupported, so the
    kernels run without IEEE NaN quieting and max() needs no
    canonicalizing moves (max reductions fuse with DPP);
  * packed fp32 instructions are switched off for the device code.

With GDNQ_SANITIZE=1 in the environment the host side of every source
(argument checks, launchers) is built with AddressSanitizer and
UndefinedBehaviorSanitizer (-Xarch_host, so device code is unchanged); the
library then needs clang's ASan runtime preloaded into the process
(sanitizer_runtime() names it).
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgdnq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "decode.hip", "window.hip", "codec.hip", "calibrate.hip", "prefill.hip", "prefill_kda.hip"]
HEADERS = ["tile.hpp", "codec.hpp", "launch.hpp", "launchers.hpp"]

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-mno-amdgpu-ieee", "-fno-honor-nans",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


SANITIZE = os.environ.get("GDNQ_SANITIZE") == "1"
# host code only: each sanitizer flag behind -Xarch_host
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def sanitizer_runtime() -> str:
    """Path of the ASan runtime of the toolchain's clang (for LD_PRELOAD)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    return subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                          text=True, check=True).stdout.strip()


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *(HOST_SANITIZE if SANITIZE else [])]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(jobs: int | None = None) -> str:
    """Compile every source and link recurrent_state_quantization_amd/libgdnq.so."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *(HOST_SANITIZE if SANITIZE else []),
                        "-Xarch_host", "-shared-libsan" if SANITIZE else "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
