"""Build libfa.so (the HIP kernels plus the C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
# The race-check build: the same library with the bf16 prefill's LDS slots poisoned before
# every refill (FA_LDS_POISON); only the race-check tests load it.
CHECK_LIB = os.path.join(PKG, "libfa_ldscheck.so")
CHECK_SOURCES = {"fa_fwd_bf16.hip": ["-DFA_LDS_POISON=1"]}
SOURCES = ["fa_api.hip", "fa_fwd_bf16.hip", "fa_fwd_f32.hip", "fa_decode.hip", "fa_bwd.hip",
           "fa_bwd_f32.hip", "fa_fwd_fp8.hip", "fa_probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
    # keep the compiler from emitting packed float32 VALU ops (v_pk_fma_f32 and kin)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # inputs with NaN are outside the contract: lets fmaxf lower to plain v_max/v_max3
    "-fno-honor-nans",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, extra=(), suffix: str = "") -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + suffix + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, lib: str):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source and link libfa.so and the race-check build libfa_ldscheck.so;
    always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(src, (), "") for src in SOURCES]
    jobs += [(src, tuple(flags), "_ldscheck") for src, flags in CHECK_SOURCES.items()]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    plain = objs[:len(SOURCES)]
    _link(plain, LIB)
    checked = {os.path.splitext(src)[0] + ".o" for src in CHECK_SOURCES}
    _link([o for o in plain if os.path.basename(o) not in checked] + objs[len(SOURCES):], CHECK_LIB)
    if verbose:
        print(f"built {LIB} and {CHECK_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
