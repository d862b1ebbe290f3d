"""Build libkvq.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m bit_kv_cache_quantize_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libkvq.so")
BUILD_DIR = os.path.join(ROOT, "_build", "kvq")

SOURCES = ["kvq_validate.cpp", "kvq_api.cpp", "quant.hip", "decode_ref.hip", "decode_mfma.hip", "decode_paged.hip",
           "decode_pruned.hip", "decode_vgroup.hip", "decode_window.hip", "stream_probe.hip", "decode_noalloc.hip"]

ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")
# -packed-fp32-ops: never emit packed fp32 VALU forms (v_pk_fma_f32 and friends).
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", f"-I{os.path.join(ROOT, 'include')}"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the kvq library needs ROCm's hipcc to build")


# per-source extra flags: keep MFMA accumulators in ordinary VGPRs (the decode kernel
# reads and rescales them with VALU code; AGPR placement would add copies)
_MFMA_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
EXTRA = {src: _MFMA_FLAGS for src in ("decode_mfma.hip", "decode_paged.hip", "decode_pruned.hip", "decode_vgroup.hip")}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *FLAGS, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"  # host pass; harmless
    msgs = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if msgs.strip():
        sys.stderr.write(msgs + "\n")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link libkvq.so next to this file. Returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build()
