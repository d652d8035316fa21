"""Compile the HIP sources into ``liblora_mi355x.so`` (the multi-LoRA path)
and ``liblora_measure.so`` (the measurement aids of lora_measure.h), gfx950.

Each ``csrc/*.hip`` file is compiled to an object in parallel, then linked
into its shared library next to this file.  Packed-FP32 instructions are
switched off for all device code.
"""

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "liblora_mi355x.so")
MEASURE_LIB = os.path.join(HERE, "liblora_measure.so")
ARCH = "gfx950"

SOURCES = ["lora_abi.hip", "metadata.hip", "metadata_grouped.hip", "shrink.hip", "expand.hip",
           "token_step.hip"]
MEASURE_SOURCES = ["stream_copy.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name: drop that note
    err = "\n".join(line for line in r.stderr.splitlines()
                    if "packed-fp32-ops" not in line or "error" in line)
    if err.strip():
        print(err, file=sys.stderr, flush=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", lib + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + MEASURE_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in MEASURE_SOURCES], MEASURE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
