"""Build libmla_host_sanitized.so: the host side of the C ABI (mla_api.cpp:
argument validation, ring and window index arithmetic, workspace carving, the
launch sequence) compiled with AddressSanitizer and UndefinedBehaviorSanitizer on
the host code only, linked with the kernel objects of the normal build.  Test
infrastructure: the ABI validation tests run against it on the CPU.

Usage: python tests/sanitize/build_host_sanitized.py   (prints the library path)
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from latent_kv_attention_down_amd import build as B  # noqa: E402

OUT_DIR = os.path.join(ROOT, "_build", "sanitize")
LIB = os.path.join(OUT_DIR, "libmla_host_sanitized.so")
# host-only instrumentation: every sanitizer flag goes to the host pass
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime():
    """The clang AddressSanitizer runtime that hipcc's host compiler links against."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang AddressSanitizer runtime not found under /opt/rocm/llvm")
    return hits[-1]


def build():
    os.makedirs(OUT_DIR, exist_ok=True)
    kernels = sorted(glob.glob(os.path.join(B.CSRC, "*.hip")))
    objs = [os.path.join(B.BUILD, os.path.basename(k) + ".o") for k in kernels]
    if not all(os.path.exists(o) for o in objs):
        B.build(verbose=False)
    api_obj = os.path.join(OUT_DIR, "mla_api.cpp.o")
    flags = [f for f in B.FLAGS if f != "-O3"] + ["-O1", "-g"]
    cmd = [B.HIPCC, *flags, *SAN, "-c", os.path.join(B.CSRC, "mla_api.cpp"), "-o", api_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized compile failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    cmd = [B.HIPCC, "-shared", "-fPIC", f"--offload-arch={B.ARCH}", "-shared-libsan", *SAN,
           "-o", LIB, api_obj, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    return LIB


if __name__ == "__main__":
    print(build())
