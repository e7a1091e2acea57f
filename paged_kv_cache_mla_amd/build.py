"""Build libkvattn.so in-tree for gfx950 with hipcc.

    python -m paged_kv_cache_mla_amd.build        (or __graft_entry__.build())
    python -m paged_kv_cache_mla_amd.build --sanitize address,undefined
    python -m paged_kv_cache_mla_amd.build --sanitize thread

The --sanitize forms build a second copy of the library, _build/san-<kinds>/libkvattn.so, whose
host code (pool, placement store, share policy, host attention, argument validation) carries
the named sanitizers; device code is compiled as usual.  Run the CPU test suite against it
with the runtime preloaded (python itself is not instrumented):

    KVATTN_LIB=_build/san-address-undefined/libkvattn.so \
    LD_PRELOAD=$(/opt/rocm/bin/hipcc -print-file-name=libclang_rt.asan-x86_64.so) \
    ASAN_OPTIONS=detect_leaks=0:halt_on_error=1 UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1 \
    python -m pytest tests -m "not gpu" -p no:cacheprovider

(`sanitizer_test_command()` prints the exact command for a build.)

Every .hip / .cpp file under csrc/ is compiled to an object in parallel and linked into
paged_kv_cache_mla_amd/libkvattn.so.  Device code is compiled with packed-fp32 instructions
disabled (-Xclang -target-feature -Xclang -packed-fp32-ops) and MFMA accumulators kept in
ordinary VGPRs (-mllvm -amdgpu-mfma-vgpr-form=1, device pass only), which avoids copies between register files
around the online-softmax rescale.
"""

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libkvattn.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]
# host code targets x86-64-v3 (AVX2 + FMA), present on every EPYC host of an MI355X; no
# implicit contraction into FMA, so scalar double arithmetic (the share policy) rounds exactly
# as written -- vector FMAs are spelled out where they are wanted
HOST_CPU = ["-mavx2", "-mfma", "-fno-math-errno", "-ffp-contract=off"]
# host files that enqueue copies use the HIP runtime API (no device code)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HOST_HIP = ["-D__HIP_PLATFORM_AMD__", "-isystem", os.path.join(ROCM, "include")]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form=1"]


def _sanitize_flags(kinds):
    """Host-side sanitizer flags for hipcc: each -fsanitize= right after -Xarch_host, so that
    only the host compilation is instrumented."""
    flags = []
    for k in kinds:
        flags += ["-Xarch_host", f"-fsanitize={k}"]
    if kinds:
        flags += ["-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
    return flags


def _compile(src: str, build_dir: str = BUILD_DIR, kinds=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    san = _sanitize_flags(kinds)
    if src.endswith(".hip"):
        cmd = [HIPCC, *COMMON, *DEVICE, *san, "-c", src, "-o", obj]
    else:  # host-only C++ (pool, host attention, share policy, placement store)
        cmd = [HIPCC, *COMMON, *HOST_CPU, *HOST_HIP, *san, "-x", "c++", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if warn:
        sys.stderr.write("\n".join(warn) + "\n")
    return obj


SANITIZERS = {"address", "undefined", "thread"}
RUNTIME = {"address": "libclang_rt.asan-x86_64.so", "thread": "libclang_rt.tsan-x86_64.so"}


def sanitized_path(kinds) -> str:
    return os.path.join(BUILD_DIR, "san-" + "-".join(kinds), "libkvattn.so")


def sanitizer_test_command(kinds) -> str:
    """The command that runs the CPU suite against the sanitized build of `kinds`."""
    rt = RUNTIME["thread" if "thread" in kinds else "address"]
    # under TSan numpy's BLAS and torch's OpenMP run on one thread: their own (uninstrumented)
    # thread pools would otherwise report races TSan cannot see the synchronisation of; the
    # library's worker threads are the ones under test
    opts = ("OPENBLAS_NUM_THREADS=1 OMP_NUM_THREADS=1 "
            "TSAN_OPTIONS='report_signal_unsafe=0 halt_on_error=1 exitcode=66'" if "thread" in kinds else
            "ASAN_OPTIONS=detect_leaks=0:halt_on_error=1 UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1")
    return (f"KVATTN_LIB={os.path.relpath(sanitized_path(kinds), ROOT)} "
            f"LD_PRELOAD=$({HIPCC} -print-file-name={rt}) {opts} "
            f"python -m pytest tests -m 'not gpu' -p no:cacheprovider")


def build(verbose: bool = True, sanitize=None) -> str:
    """Compile every source and link the library.  sanitize: None for the product library,
    or an iterable of "address" / "undefined" / "thread" for the sanitized copy."""
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    kinds = tuple(sorted(sanitize or ()))
    if set(kinds) - SANITIZERS or ("thread" in kinds and len(kinds) > 1):
        raise ValueError(f"sanitize: address and/or undefined, or thread alone; got {kinds}")
    out = sanitized_path(kinds) if kinds else OUT
    build_dir = os.path.dirname(out) if kinds else BUILD_DIR
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, kinds), srcs))
    tmp = out + ".tmp"
    # a sanitized library leaves the runtime's symbols to the preloaded runtime
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-lpthread", "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
        if kinds:
            print("run the CPU suite against it with:\n  " + sanitizer_test_command(kinds))
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="build libkvattn.so for gfx950")
    ap.add_argument("--sanitize", default="",
                    help="comma-separated host sanitizers: address,undefined or thread")
    args = ap.parse_args()
    build(sanitize=[k for k in args.sanitize.split(",") if k] or None)
