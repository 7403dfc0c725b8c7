"""Build libbsa.so (the gfx950 kernels + the C ABI) in-tree with hipcc.

    python -m content_dependent_block_amd.build

Every HIP source is compiled for gfx950 only, with packed-FP32 instruction
selection turned off (-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
OBJ = PKG / "_build"
LIB = PKG / "libbsa.so"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["block_pool.hip", "coarse_score.hip", "topk_select.hip", "sparse_flash_fwd.hip",
           "fine_gather.hip", "fine_backward.hip", "ragged.hip", "noalloc.hip", "bsa_api.cpp", "tiles.cpp"]

FLAGS = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wno-unused-result", f"-I{ROOT / 'include'}", f"-I{CSRC}"]


# Per-source extras.  coarse_score and fine_gather: their scores are never
# NaN for finite inputs, and without NaN semantics a max of MFMA results
# needs no canonicalising instruction in front of it.  (fine_gather's one
# documented non-finite case, a bf16 value beyond the fp16 range, reaches the
# output through the combine's multiply-adds, which propagate inf and NaN
# whatever the flag.)
EXTRA = {"coarse_score.hip": ["-fno-honor-nans"], "fine_gather.hip": ["-fno-honor-nans"]}


def _compile(src: str) -> Path:
    out = OBJ / (src + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", str(CSRC / src), "-o", str(out)]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return out


def build(jobs: int | None = None) -> Path:
    OBJ.mkdir(exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 8)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB.with_suffix(".so.tmp")
    r = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", str(tmp),
                        *map(str, objs)], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(int(sys.argv[1]) if len(sys.argv) > 1 else None))
