"""Build the gfx950 HIP library in-tree: libtessera_attn.so beside this file
(the attention forward and backward, paged decode, and the fused RMSNorm).

    python -m attention_flashattention_fwd_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
SOURCES = [PKG / "csrc" / "tessera_attn.hip", PKG / "csrc" / "tessera_attn_bwd.hip",
           PKG / "csrc" / "tessera_rmsnorm.hip", PKG / "csrc" / "tessera_paged.hip"]
INCLUDE = ROOT / "include"
LIBRARY = PKG / "libtessera_attn.so"
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # no NaN handling in max/min: inputs are finite by contract, and masked
    # scores are -inf, never NaN
    "-fno-honor-nans",
    # packed fp32 vector ops stay off: the kernels are written for scalar fp32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def build(verbose: bool = False, extra: list[str] | None = None) -> Path:
    tmp = LIBRARY.with_suffix(".so.tmp")
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra or []), f"-I{INCLUDE}", *map(str, SOURCES), "-o",
           str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the fp32 feature flag and says so; drop that line
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
