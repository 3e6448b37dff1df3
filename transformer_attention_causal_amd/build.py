"""Build libattn.so (the HIP kernels and the C ABI) for gfx950, in place, with hipcc.

    python -m transformer_attention_causal_amd.build [--verbose] [--resource-usage] [--asan]

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

# Per-source flags. decode.hip: MFMA accumulators in ordinary VGPRs (the multi-head 8-bit kernel otherwise splits
# its registers over VGPRs and AGPRs, drops to one wave per SIMD, and moves accumulators between the two files).
SOURCE_FLAGS = {"decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: ROCm is required to build libattn")
    return path


def _compile(src, verbose, extra):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
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


ASAN_DIR = os.path.join(BUILD_DIR, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libattn_asan.so")


def asan_runtime():
    """Path of the AddressSanitizer runtime of ROCm's clang (to preload into a host process)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = shutil.which("clang") or "clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang's AddressSanitizer runtime was not found")
    return path


def build_asan(verbose=False):
    """A build of libattn whose host code in capi.hip (the C ABI's argument validation) is compiled with
    AddressSanitizer; the device code and the other sources are the normal build's objects. For CPU tests of
    the C ABI only: load it into a process that preloads asan_runtime()."""
    if not all(os.path.exists(os.path.join(BUILD_DIR, os.path.splitext(f)[0] + ".o")) for f in SOURCES):
        build(verbose)
    os.makedirs(ASAN_DIR, exist_ok=True)
    obj = os.path.join(ASAN_DIR, "capi.o")
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    cmd = [hipcc(), *HIPCC_FLAGS, *host_asan, "-c", os.path.join(CSRC, "capi.hip"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the ASan build:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    objs = [obj] + [os.path.join(BUILD_DIR, os.path.splitext(f)[0] + ".o") for f in SOURCES if f != "capi.hip"]
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-shared-libasan", "-o", ASAN_LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"ASan link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    return ASAN_LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true", help="print per-kernel register/LDS usage")
    ap.add_argument("--asan", action="store_true", help="also build the host-ASan variant of the C ABI (CPU tests)")
    args = ap.parse_args()
    print(build(verbose=args.verbose, resource_usage=args.resource_usage))
    if args.asan:
        print(build_asan(verbose=args.verbose))
    sys.exit(0)
