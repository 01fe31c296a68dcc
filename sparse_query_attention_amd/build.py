"""Build libsqa.so in-tree with hipcc for gfx950 (cross-compiles without a GPU).

    python -m sparse_query_attention_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["sqa_api.hip", "sqa_gemm.hip", "sqa_attention.hip", "sqa_decode.hip", "sqa_backward.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU forms stay off: the kernels are written for scalar fp32 math
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build_library(verbose: bool = True) -> str:
    out = os.path.join(HERE, "libsqa.so")
    tmp = out + f".tmp{os.getpid()}"
    cmd = [HIPCC, *FLAGS, f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(HERE, 'csrc')}",
           *[os.path.join(HERE, "csrc", s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name; that note is harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.unlink(tmp)
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library())
