"""Build libxs.so in-tree with hipcc for gfx950.

    python -m paged_kv_decode_xs_amd.build          # compile every source, link libxs.so

Each csrc/*.hip file compiles to an object in _build/ (in parallel), then the objects link into
paged_kv_decode_xs_amd/libxs.so. The build always recompiles: it is the "does it build" check.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
from typing import List, Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
BUILD_DIR = os.path.join(REPO_DIR, "_build", "libxs")
LIB_PATH = os.path.join(PKG_DIR, "libxs.so")

ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # Code object v5 loads in both the ROCm 7.0 runtime that torch bundles and ROCm 7.2.
    "-mcode-object-version=5",
    # No packed fp32 instructions (v_pk_fma_f32 and friends) anywhere in device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", INCLUDE,
    "-I", CSRC,
]


# Per-source additions. The prefill attention keeps its MFMA accumulators in VGPRs (it rescales
# them with vector ALU ops); the default heuristic puts them in AGPRs and copies them around
# every matrix op.
FILE_FLAGS = {
    "xs_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    env = os.environ.get("HIPCC")
    if env:
        return env
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def sources() -> List[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd: List[str]) -> None:
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out, file=sys.stderr)


def build(verbose: bool = False, jobs: Optional[int] = None) -> str:
    """Compile all sources and link libxs.so. Returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    srcs = sources()
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    cmds = [[cc, *COMMON_FLAGS, *FILE_FLAGS.get(os.path.basename(s), []), "-c", s, "-o", o]
            for s, o in zip(srcs, objs)]
    jobs = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for cmd, fut in [(c, ex.submit(_run, c)) for c in cmds]:
            if verbose:
                print(" ".join(cmd), file=sys.stderr)
            fut.result()
    tmp = LIB_PATH + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the library: the host code is
# instrumented (each -fsanitize= behind -Xarch_host), the device code is built as usual. It
# exists to run the C-ABI checks (tests/test_abi.py) on the CPU under the sanitizers; load it with
# the ASan runtime preloaded (sanitizer_env()). It is never loaded on a GPU.
SAN_DIR = os.path.join(REPO_DIR, "_build", "asan")
SAN_LIB = os.path.join(SAN_DIR, "libxs.so")
SAN_FLAGS = [
    f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-mcode-object-version=5", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
    "-I", INCLUDE, "-I", CSRC,
]


def asan_runtime() -> str:
    """The clang ASan runtime that matches hipcc (preloaded into the process that loads SAN_LIB)."""
    import glob

    root = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "llvm", "lib", "clang")
    hits = sorted(glob.glob(os.path.join(root, "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not hits:
        hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang ASan runtime not found")
    return hits[-1]


def build_host_sanitized(jobs: Optional[int] = None) -> str:
    """Compile every source's host code with ASan and UBSan and link SAN_LIB. Returns its path."""
    os.makedirs(SAN_DIR, exist_ok=True)
    cc = hipcc()
    srcs = sources()
    objs = [os.path.join(SAN_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    cmds = [[cc, *SAN_FLAGS, *FILE_FLAGS.get(os.path.basename(s), []), "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    jobs = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for fut in [ex.submit(_run, c) for c in cmds]:
            fut.result()
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", "-shared-libasan", *objs, "-o", SAN_LIB])
    return SAN_LIB


def sanitizer_env() -> dict:
    """Environment for a child process that loads SAN_LIB (through XS_LIBRARY)."""
    env = dict(os.environ)
    env["XS_LIBRARY"] = SAN_LIB
    env["LD_PRELOAD"] = asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=87"
    return env


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized())
    else:
        print(build(verbose="-v" in sys.argv))
