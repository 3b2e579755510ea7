"""Build libpagedattn.so (HIP for gfx950) in-tree.

    python -m decode_attention_paged_append_amd.build

Each source compiles to an object under _build/ in parallel; the objects are
then linked into decode_attention_paged_append_amd/libpagedattn.so.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libpagedattn.so")

SOURCES = ["api.cpp", "block_manager.cpp", "kv_ops.hip", "lse_merge.hip", "noalloc.hip",
           "decode_f32.hip",
           "decode_f16.hip", "decode_bf16.hip", "decode_i8.hip", "decode_fp8.hip",
           "decode_i4.hip",
           "prefill_f16.hip",
           "prefill_bf16.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions: hipcc would otherwise form v_pk_*_f32 itself
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE binary32 division and square root (the int8 quantizer divides)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-file additions.  The prefill kernels keep their matrix-core
# accumulators in VGPRs: in the AGPR form the backend copied all 128 of them
# AGPR -> VGPR on every tile of the KV loop.
EXTRA_FLAGS = {
    "prefill_f16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "prefill_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIBRARY + ".tmp"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build())
