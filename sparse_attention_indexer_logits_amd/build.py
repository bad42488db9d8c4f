"""Build libxk.so (gfx950) in-tree with hipcc.

    python sparse_attention_indexer_logits_amd/build.py

Every HIP source is compiled with packed-fp32 VALU ops disabled
(-target-feature -packed-fp32-ops); hipcc's host pass warns that it does not
know that feature, which is harmless.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libxk.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc") or ""):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm 7.x expected under /opt/rocm)")


# Extra flags per source. The logits kernel feeds MFMA accumulators into
# ReLU; without NaN-honoring, max(x, 0) is one v_max_f32 instead of a
# canonicalize + max (NaN inputs are outside the C ABI contract anyway).
PER_SOURCE_FLAGS = {"logits.hip": ["-fno-honor-nans"]}
COMMON = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
NOISE = "is not a recognized feature for this target"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if NOISE not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def build(verbose: bool = False) -> str:
    from concurrent.futures import ThreadPoolExecutor

    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    jobs = []
    for src in srcs:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        flags = PER_SOURCE_FLAGS.get(os.path.basename(src), [])
        jobs.append((obj, [hipcc()] + COMMON + flags + inc + ["-c", src, "-o", obj]))
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda j: _run(j[1], verbose), jobs))
    tmp = LIB + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [j[0] for j in jobs],
         verbose)
    os.replace(tmp, LIB)
    # the benchmark's achievable-rate probes: a library of their own
    peaks = os.path.join(PKG, "libxk_peaks.so")
    _run([hipcc()] + COMMON + ["-shared", "-o", peaks + ".tmp", os.path.join(PKG, "probes", "peaks.hip")], verbose)
    os.replace(peaks + ".tmp", peaks)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
