"""Build libnvfp4moe.so (the HIP library behind include/nvfp4moe.h) for gfx950, in-tree.

Each csrc/*.hip is compiled to an object in parallel, then linked into one shared library. Flags:
  --offload-arch=gfx950                   MI355X only
  -ffp-contract=off                       every FP multiply/add is rounded as written (the
                                          reduction order in nvfp4_device.hpp is part of the contract)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                          no packed FP32 instructions are generated
  -fvisibility=hidden                     only the extern "C" entry points are exported
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libnvfp4moe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-command-line-argument"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC] + CFLAGS + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


SAN_LIB = os.path.join(BUILD, "san", "libnvfp4moe_san.so")


def build_host_sanitized(verbose: bool = False) -> str:
    """A host-sanitizer build of the library for the host-side checks (tests/test_sanitizers.py):
    abi.hip, which holds every argument check, compiled with AddressSanitizer and
    UndefinedBehaviorSanitizer on its host code only (the device code is built as usual), linked
    with the regular objects of the other sources. Loaded into a Python that preloads clang's ASan
    runtime; it is never launched on a GPU."""
    if not all(os.path.exists(os.path.join(BUILD, n)) for n in ("linear.o", "moe_gemm.o", "moe_plan.o",
                                                                 "moe_prefill.o")):
        build(verbose)
    san = os.path.join(BUILD, "san")
    os.makedirs(san, exist_ok=True)
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
    obj = os.path.join(san, "abi.o")
    cmd = [HIPCC] + CFLAGS + host_san + ["-c", os.path.join(CSRC, "abi.hip"), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for abi.hip (host sanitizers):\n{r.stderr}")
    others = [os.path.join(BUILD, n) for n in ("linear.o", "moe_gemm.o", "moe_plan.o", "moe_prefill.o")]
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", SAN_LIB, obj] + others
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return SAN_LIB


if __name__ == "__main__":
    print(build_host_sanitized(verbose=True) if "--sanitize-host" in sys.argv else build(verbose="-v" in sys.argv))
