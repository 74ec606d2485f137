"""Build libllatte.so (HIP for gfx950) in place, next to this file.

    python -m target_aware_latent_amd.build              # the library
    python -m target_aware_latent_amd.build --sanitize   # host-instrumented copy

Every .hip source under csrc/ is compiled with hipcc for gfx950 and linked
into one shared library with a C ABI (declared in include/llatte.h).

--sanitize builds a second copy under _build/sanitize/ whose HOST code
(validation, workspace planning, orchestration) carries AddressSanitizer and
UndefinedBehaviorSanitizer; the device code is compiled as usual. Load it
with LLATTE_LIBRARY=<path> and the ASan runtime preloaded (asan_runtime()).
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libllatte.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function",
]
# Per-source extras. The attention kernels never produce NaN on valid input
# (masked scores are -inf, every query row sees at least one key), so max
# needs no NaN quieting and the IEEE-mode canonicalisation can go.
FILE_FLAGS = {
    "attention.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
}


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip"))


# host-only instrumentation: each -fsanitize= applies to the host pass alone
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
SAN_DIR = os.path.join(BUILD, "sanitize")


def asan_runtime():
    """Path of the ASan runtime that a sanitized library needs preloaded."""
    res = subprocess.run([HIPCC.replace("hipcc", "amdclang++"),
                          "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    return res.stdout.strip()


def _compile(src, verbose, out_dir=BUILD, extra=()):
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src,
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = (res.stdout + res.stderr).replace(
        "'-packed-fp32-ops' is not a recognized feature for this target "
        "(ignoring feature)\n", "")
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    return obj


def build(verbose=False, sanitize=False):
    """Compile every HIP source and link libllatte.so; returns its path.
    With sanitize the host-instrumented copy is built under _build/sanitize/."""
    out_dir = SAN_DIR if sanitize else BUILD
    lib = os.path.join(SAN_DIR, "libllatte.so") if sanitize else LIB
    extra = SAN_FLAGS if sanitize else ()
    os.makedirs(out_dir, exist_ok=True)
    srcs = _sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, out_dir, extra), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", *extra, "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
