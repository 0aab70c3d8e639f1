"""Build libkara.so (the Kara library) and libkara_probes.so (achievable-peak
probes used by the measurements) in-tree with hipcc for gfx950.

    python -m decode_kv_cache_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkara.so")
SOURCES = ["api.hip", "score.hip", "score_fused.hip", "score_small.hip", "select.hip", "compact.hip",
           "decode_attn.hip"]
PROBES_LIB = os.path.join(PKG, "libkara_probes.so")
PROBES_SOURCES = ["probes.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the softmax arithmetic reads them directly
    # instead of copying each one out of an AGPR first
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # scores, logits and weights are never NaN: max/min need no quieting of
    # their operands (infinities stay honoured; the kernels rely on them)
    "-fno-honor-nans",
    "-Wno-unused-result",
]
# roctx ranges around the entry points (host-side trace markers)
HIPCC_LIBS = ["-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = True, out: str = LIB, csrc: str = CSRC, extra=(), sources=None) -> str:
    """Compile the library's HIP sources into libkara.so next to this file
    (and the probes into libkara_probes.so); return the library's path."""
    if out == LIB and sources is None:
        _compile(verbose, PROBES_LIB, csrc, extra, PROBES_SOURCES)
    return _compile(verbose, out, csrc, extra, sources or SOURCES)


def _compile(verbose, out, csrc, extra, sources) -> str:
    tmp = out + ".tmp"
    libs = HIPCC_LIBS if "api.hip" in sources else []
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, f"-I{INCLUDE}", f"-I{csrc}",
           *[os.path.join(csrc, s) for s in sources], *libs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build()
