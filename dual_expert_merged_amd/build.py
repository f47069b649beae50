"""Build libdm.so (HIP, gfx950) in-tree with hipcc.  ``python -m dual_expert_merged_amd.build``."""
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdm.so")
SOURCES = ["dm_api.cpp", "gemm.hip", "attn.hip", "misc.hip", "persist.hip", "train.hip"]
# attention rescales its MFMA accumulators with VALU every key tile: keep them in VGPRs rather
# than accumulation registers, which would cost a copy out and back per element.  Its softmax
# takes many float maxima of MFMA results that are never NaN: without -fno-honor-nans every
# fmaxf operand is first canonicalised (an extra instruction each).
EXTRA = {"attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"]}

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-I" + os.path.join(ROOT, "include"),
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdm)")


def build(verbose=False):
    """Compile every HIP/C++ source into libdm.so (always recompiles)."""
    objs = []
    procs = []
    t0 = time.time()
    tmpdir = os.path.join(PKG, "_build")
    os.makedirs(tmpdir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(tmpdir, src + ".o")
        flags = [f for f in HIPCC_FLAGS if f != "-shared"]
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [hipcc()] + flags + EXTRA.get(src, []) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = False
    for src, cmd, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        noise = "is not a recognized feature for this target"
        text = "\n".join(line for line in text.splitlines() if noise not in line)
        if p.returncode != 0:
            failed = True
            sys.stderr.write(f"[build] {src} failed:\n{' '.join(cmd)}\n{text}\n")
        elif verbose and text.strip():
            sys.stderr.write(f"[build] {src}:\n{text}\n")
    if failed:
        raise RuntimeError("libdm build failed")
    tmp = LIB + ".tmp"
    link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.run(link, check=True)
    os.replace(tmp, LIB)
    if verbose:
        sys.stderr.write(f"[build] {LIB} in {time.time() - t0:.1f}s\n")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
