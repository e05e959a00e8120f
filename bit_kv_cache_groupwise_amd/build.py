"""Build libkvq.so (HIP kernels for gfx950 + the C-ABI host library) in-tree.

    python -m bit_kv_cache_groupwise_amd.build

Every call recompiles. Flags that matter for the numerics: no FP contraction
(the quantizer's subtract and divide must not fuse), correctly rounded fp32
division, fp32 denormals kept; packed fp32 VALU ops are disabled.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvq.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")

MHA_HEAD_DIMS = (64, 128, 256)
GQA_ROPE_HEAD_DIMS = (128, 256)  # rotary keys on the query-group kernel
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
DEVICE = [f"--offload-arch={ARCH}", "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
          "-fno-gpu-flush-denormals-to-zero", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    return os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def units():
    """(source, object, extra flags, is_device_code) of every translation unit."""
    return [("kvq_kernels.hip", "kvq_kernels.o", [], True),
            ("kvq_scratch.hip", "kvq_scratch.o", [], True),
            *[("kvq_decode_mha.hip", f"kvq_decode_mha_d{d}.o", [f"-DKVQ_MHA_HEAD_DIM={d}"], True)
              for d in MHA_HEAD_DIMS],
            *[("kvq_decode_mha.hip", f"kvq_decode_mha_rope_d{d}.o", [f"-DKVQ_MHA_HEAD_DIM={d}", "-DKVQ_MHA_ROPE=1"], True)
              for d in MHA_HEAD_DIMS],
            *[("kvq_decode_gqa.hip", f"kvq_decode_gqa_d{d}.o", [f"-DKVQ_GQA_HEAD_DIM={d}"], True)
              for d in MHA_HEAD_DIMS],
            *[("kvq_decode_gqa.hip", f"kvq_decode_gqa_rope_d{d}.o", [f"-DKVQ_GQA_HEAD_DIM={d}", "-DKVQ_GQA_ROPE=1"], True)
              for d in GQA_ROPE_HEAD_DIMS],
            ("kvq_api.cpp", "kvq_api.o", [], False)]


def _compile_cmd(cc, src, obj, extra, device):
    out = os.path.join(BUILD, obj)
    if device:
        return [cc, *COMMON, *DEVICE, *extra, "-c", os.path.join(CSRC, src), "-o", out]
    return [cc, *COMMON, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), *extra, "-c",
            os.path.join(CSRC, src), "-o", out]


def link() -> str:
    cc = hipcc()
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
          *[os.path.join(BUILD, u[1]) for u in units()]])
    os.replace(tmp, LIB)
    return LIB


def build_host_sanitized(out_dir: str) -> str:
    """libkvq with its host code (argument checks, layout, page management)
    built by g++ under AddressSanitizer and UndefinedBehaviorSanitizer, linked
    with this build's device objects (which must exist: build() first). For the
    CPU tests of the C ABI; load it with libasan preloaded."""
    os.makedirs(out_dir, exist_ok=True)
    obj = os.path.join(out_dir, "kvq_api_sanitized.o")
    lib = os.path.join(out_dir, "libkvq_sanitized.so")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    _run(["g++", "-O1", "-g", "-std=c++17", "-fPIC", *san, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
          "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, "kvq_api.cpp"), "-o", obj])
    devobjs = [os.path.join(BUILD, u[1]) for u in units() if u[3]]
    _run(["g++", "-shared", *san, "-o", lib, obj, *devobjs, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"])
    return lib


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    jobs = [_compile_cmd(cc, *u) for u in units()]
    with ThreadPoolExecutor(min(len(jobs), os.cpu_count() or 4)) as ex:
        for r in ex.map(_run, jobs):
            if verbose and (r.stdout or r.stderr):
                print(r.stdout, r.stderr, file=sys.stderr)
    return link()


if __name__ == "__main__":
    print(build(verbose=True))
