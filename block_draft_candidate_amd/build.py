"""Build libdflash.so (HIP, gfx950) in-tree with hipcc.

    python -m block_draft_candidate_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdflash.so")
SOURCES = ["lm_topk.hip", "edges.hip", "qk_norm_rope.hip", "block_attn.hip", "context_kv.hip", "linear.hip", "api.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Wno-unused-function",
    # never let the compiler form packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


# Per-source extra flags.  Attention rescales its MFMA accumulators with VALU
# work every tile; with the default AGPR form they are copied AGPR <-> VGPR
# around that, so the MFMAs there are kept in their VGPR form.
EXTRA_FLAGS = {"block_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdflash.so)")


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libdflash.so next to this
    file.  Always recompiles.  Returns the library path."""
    hipcc = _hipcc()
    tmp = tempfile.mkdtemp(prefix="dflash_build_")
    try:
        def compile_one(src: str) -> str:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [hipcc, *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
            res = subprocess.run(cmd, capture_output=True, text=True)
            noise = "is not a recognized feature for this target"
            err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{err}")
            if verbose and err.strip():
                print(err, file=sys.stderr)
            return obj

        with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        out_tmp = LIB + ".tmp"
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp, *objs]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stderr}")
        os.replace(out_tmp, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
