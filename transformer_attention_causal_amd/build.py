"""Build libattn.so (the HIP kernels and the C ABI) for gfx950, in place, with hipcc.

    python -m transformer_attention_causal_amd.build [--verbose]

Every HIP source is compiled with -Xclang -target-feature -Xclang -packed-fp32-ops (no packed fp32 ops are
generated) and the objects are linked into transformer_attention_causal_amd/libattn.so. hipcc cross-compiles, so
no GPU is needed to build.
"""
import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn.so")
SOURCES = ["rope.hip", "prefill.hip", "decode.hip", "mla.hip", "dsa.hip", "capi.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-I", os.path.join(ROOT, "include"),
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: ROCm is required to build libattn")
    return path


def _compile(src, verbose, extra):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "is not a recognized feature for this target" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def build(verbose=False, resource_usage=False):
    """Compile every HIP source for gfx950 and link libattn.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    with ThreadPoolExecutor(min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose or resource_usage, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true", help="print per-kernel register/LDS usage")
    args = ap.parse_args()
    print(build(verbose=args.verbose, resource_usage=args.resource_usage))
    sys.exit(0)
