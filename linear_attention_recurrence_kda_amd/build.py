"""Build the KDA HIP library (libkda.so) in-tree for gfx950 with hipcc.

Usage:  python -m linear_attention_recurrence_kda_amd.build [-v]
Every source under csrc/ is compiled to an object in _build/ (at the repo
root) and linked into linear_attention_recurrence_kda_amd/libkda.so.
"""
import concurrent.futures as cf
import glob
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkda.so")
ARCH = "gfx950"

# Packed fp32 instructions are kept out of the generated code (-packed-fp32-ops).
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]


def _hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found; the KDA library needs ROCm's hipcc")
    return h


# Per-source additions: the column-slab kernel keeps MFMA results in ordinary
# vector registers (it rescales and rounds them every chunk).
EXTRA = {"kda_slab.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "kda_fused.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}

# Sources whose kernels must not use scratch memory: a spill or a
# dynamically indexed private array there costs a memory round trip per
# chunk on the longest chain (and its vmcnt waits hold every load in flight),
# so the build fails instead of shipping a silently slower kernel.
NO_SCRATCH = {"kda_fused.hip", "kda_slab.hip", "kda_cp.hip"}
_SCRATCH_RE = re.compile(r"ScratchSize \[bytes/lane\]: (\d+)")
_NAME_RE = re.compile(r"Function Name: (\S+)")


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    base = os.path.basename(src)
    cmd = [_hipcc()] + COMMON + EXTRA.get(base, []) + ["-c", src, "-o", obj]
    if base in NO_SCRATCH:
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if base in NO_SCRATCH:
        name = "?"
        for line in r.stderr.splitlines():
            m = _NAME_RE.search(line)
            if m:
                name = m.group(1)
            m = _SCRATCH_RE.search(line)
            if m and int(m.group(1)) != 0:
                raise RuntimeError(f"{base}: kernel {name} uses {m.group(1)} bytes of scratch per lane")
    if verbose and r.stderr.strip():
        print(r.stderr, flush=True)
    return obj


def build(verbose=False):
    """Compile every source and link libkda.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
