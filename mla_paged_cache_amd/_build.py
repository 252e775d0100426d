"""Build the gfx950 library libleyline.so in-tree with hipcc.

The library holds the HIP kernels (csrc/kernels.hip for MLA pools,
csrc/kernels_gqa.hip for GQA / MHA pools, csrc/kernels_kvs.hip for the
KV-streams trainer mask, csrc/kernels_rows.hip for the per-row-angle
rotation, csrc/kernels_alloc.hip for the eviction's device-side page
allocator, helpers in csrc/device_common.h) and the C++ host
side and C ABI (csrc/pool.cpp, csrc/kvs_mask.cpp).  Flags:
  * --offload-arch=gfx950 only (MI355X);
  * -ffp-contract=off so the delta-rotation keeps its separately rounded
    float32 products (the kernels also say so with a pragma);
  * -target-feature -packed-fp32-ops keeps the compiler away from packed fp32
    instructions.
"""

from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libleyline.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = [os.path.join(CSRC, n) for n in ("kernels.hip", "kernels_gqa.hip", "kernels_kvs.hip", "kernels_rows.hip",
                                           "kernels_alloc.hip", "pool.cpp", "kvs_mask.cpp")]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Winfinite-recursion",
    "-Wl,--no-undefined",
    # host code: the hardware popcount (the free-page bitmap is merged and
    # counted word by word; without it every popcount is a dozen ALU ops)
    "-Xarch_host", "-mpopcnt",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


def build(verbose: bool = False) -> str:
    """Compile libleyline.so next to this file; returns its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", INCLUDE, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l and "ignoring feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
