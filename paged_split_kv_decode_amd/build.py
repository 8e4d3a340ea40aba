"""Builds the HIP library ``libpaged_decode.so`` in-tree for gfx950.

Every ``csrc/*.hip`` file is compiled with hipcc (packed-FP32 instructions
disabled) and linked into one shared library next to this file.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
OBJ_DIR = os.path.join(REPO_DIR, "_build", "obj")
LIB_NAME = "libpaged_decode.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = os.environ.get("PD_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    "-I", os.path.join(REPO_DIR, "include"),
]


def _hipcc() -> str:
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return cand if os.path.exists(cand) else (shutil.which("hipcc") or "hipcc")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Per-source code-generation flags.  The MLA kernel keeps its 256 x 32 fp32
# accumulator per wave in AGPRs so the VGPR file holds the query fragment
# and the LDS operands.  The GQA kernel's accumulator (8 x 4 fp32 per lane)
# is rescaled by the softmax every tile: with the MFMA results in VGPRs it
# needs no AGPR copies in and out around each product (FP8 cache: 6-7% less
# time per call).
PER_SOURCE_FLAGS = {
    "mla_verify.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=0"],
    "mla_verify_small_pages.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=0"],
    "mla_verify_general_pages.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=0"],
    "gqa_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "gqa_decode_small_pages.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "gqa_decode_general_pages.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "gqa_append.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "gqa_append_small_pages.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    per = PER_SOURCE_FLAGS.get(os.path.basename(src), [])
    cmd = [_hipcc(), *HIPCC_FLAGS, *per, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(extra_flags: list[str] | None = None, jobs: int = 8) -> str:
    """Compile and link the library; returns the path of the .so."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    extra = list(extra_flags or [])
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), sources()))
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
    sys.exit(0)
