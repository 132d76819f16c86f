"""Build libmla_decode.so in place with hipcc for gfx950.

Every source under csrc/ is compiled to an object in _build/ (in parallel), then
linked into mla_latent_kv_03_amd/libmla_decode.so.  Run ``python -m
mla_latent_kv_03_amd.build`` or call ``build()``.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libmla_decode.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["mla_api.cpp", "mla_proj_api.cpp", "mla_attn_mfma.hip", "mla_attn_h128.hip", "mla_attn_fp8_v0.hip",
           "mla_attn_f32.hip", "mla_combine.hip", "mla_append.hip", "mla_proj.hip", "mla_gqla.hip"]
ARCH = "gfx950"


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libmla_decode.so")
    return path


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed FP32 instructions are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *compile_flags(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


PEAKS_SRC = os.path.join(PKG, "peaks", "mla_peaks.hip")
PEAKS_LIB = os.path.join(PKG, "peaks", "libmla_peaks.so")


def build_peaks(verbose=False):
    """The attainable-peak probes (bench.py --peaks), a library of their own."""
    tmp = PEAKS_LIB + ".tmp"
    cmd = [hipcc(), *compile_flags(), "-shared", "-x", "hip", PEAKS_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on mla_peaks.hip:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, PEAKS_LIB)
    return PEAKS_LIB


def build(verbose=False):
    """Compile every HIP source for gfx950 and link libmla_decode.so (always rebuilds), and the
    peak probes."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    build_peaks(verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
