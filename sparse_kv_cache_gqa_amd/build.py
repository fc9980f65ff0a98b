"""Build libda.so (HIP kernels for gfx950 + the C ABI) in-tree.

    python -m sparse_kv_cache_gqa_amd.build [-v] [-j N]

Objects go to <repo>/_build/, the library to sparse_kv_cache_gqa_amd/libda.so.
Every source is compiled on every call (this is the "does it build" check as
well as the build).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libda.so")

SOURCES = [
    "csrc/api.cpp",
    "csrc/stream.cpp",
    "csrc/kernels/attn.hip",
    "csrc/kernels/attn_u4.hip",
    "csrc/kernels/page.hip",
    "csrc/kernels/kv4.hip",
    "csrc/kernels/prefill.hip",
    "csrc/kernels/append.hip",
    "csrc/kernels/read_stream.hip",
]

ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libda.so)")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
        # keep fp32 arithmetic off the packed-fp32 (v_pk_*_f32) instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-I", os.path.join(PKG, "csrc"),
    ]


# Per-source compiler options on top of common_flags().
EXTRA_FLAGS = {
    # uint4 partial pass: MFMA accumulators in VGPRs (no AGPR copies per stage)
    "csrc/kernels/attn_u4.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, verbose: bool, out_dir: str = BUILD) -> str:
    path = os.path.join(PKG, src)
    obj = os.path.join(out_dir, src.replace("/", "_") + ".o")
    cmd = [hipcc(), *common_flags(), *EXTRA_FLAGS.get(src, []), "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host-sanitizer build: the C-ABI layer (argument checks, streaming driver)
# under AddressSanitizer and UndefinedBehaviorSanitizer, for checking on the
# CPU.  The host files are compiled by g++ (host code only); the kernels are
# compiled as usual and linked in unchanged.  Loading it into a process needs
# the ASan runtime preloaded (see tests/test_abi_sanitized.py).
HOST_SOURCES = ["csrc/api.cpp", "csrc/stream.cpp"]
SAN_DIR = os.path.join(BUILD, "host_sanitize")
SAN_LIB = os.path.join(SAN_DIR, "libda_hostsan.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def rocm_root() -> str:
    return os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))


def build_host_sanitized(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(SAN_DIR, exist_ok=True)
    rocm = rocm_root()
    kernels = [s for s in SOURCES if s not in HOST_SOURCES]

    def host_obj(src: str) -> str:
        obj = os.path.join(SAN_DIR, src.replace("/", "_") + ".o")
        cmd = ["g++", "-std=c++17", "-fPIC", "-O1", "-g", *SAN_FLAGS, "-D__HIP_PLATFORM_AMD__",
               "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
               "-I", os.path.join(PKG, "csrc"), "-c", os.path.join(PKG, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {src}\n{r.stderr}")
        return obj

    jobs = jobs or min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        kobjs = list(ex.map(lambda s: _compile(s, verbose, SAN_DIR), kernels))
        hobjs = list(ex.map(host_obj, HOST_SOURCES))
    tmp = SAN_LIB + ".tmp"
    cmd = ["g++", "-shared", *SAN_FLAGS, "-o", tmp, *hobjs, *kobjs, "-L", os.path.join(rocm, "lib"),
           "-lamdhip64", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("-j", "--jobs", type=int, default=None)
    ap.add_argument("--host-sanitize", action="store_true",
                    help="also build the host-sanitizer variant (ASan + UBSan on the C-ABI layer)")
    a = ap.parse_args(argv)
    print(build(a.verbose, a.jobs))
    if a.host_sanitize:
        print(build_host_sanitized(a.verbose, a.jobs))
    return 0


if __name__ == "__main__":
    sys.exit(main())
