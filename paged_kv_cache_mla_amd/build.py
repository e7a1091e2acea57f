"""Build libkvattn.so in-tree for gfx950 with hipcc.

    python -m paged_kv_cache_mla_amd.build        (or __graft_entry__.build())

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


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC, *COMMON, *DEVICE, "-c", src, "-o", obj]
    else:  # host-only C++ (pool, host attention, share policy, placement store)
        cmd = [HIPCC, *COMMON, *HOST_CPU, *HOST_HIP, "-x", "c++", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if warn:
        sys.stderr.write("\n".join(warn) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-lpthread", "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build()
