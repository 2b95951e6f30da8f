"""Host-side sanitizer run of the library's C ABI layer (CPU only).

Usage:  python -m linear_attention_recurrence_kda_amd.sanitize

Builds a copy of the library with AddressSanitizer and UndefinedBehavior-
Sanitizer on its host code (every hipcc line takes the sanitizer flags behind
-Xarch_host, so device code is built as usual) into _build/asan/, then runs
the CPU tests of the C ABI (tests/test_abi.py: argument validation, error
paths, plan queries, exported symbols) against it with the clang ASan runtime
preloaded.  Exits with the test run's status.
"""
import glob
import os
import subprocess
import sys

from . import build as B

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
       "-Xarch_host", "-shared-libsan"]


def asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang's ASan runtime (libclang_rt.asan-x86_64.so) not found under /opt/rocm")
    return hits[-1]


def build_sanitized(verbose=False):
    out = os.path.join(B.BUILD, "asan")
    os.makedirs(out, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(B.CSRC, "*.hip")) + glob.glob(os.path.join(B.CSRC, "*.cpp")))
    objs = []
    for src in srcs:
        obj = os.path.join(out, os.path.basename(src) + ".o")
        cmd = [B._hipcc()] + B.COMMON + SAN + B.EXTRA.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = ["-x", "hip"]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        objs.append(obj)
    lib = os.path.join(out, "libkda_asan.so")
    cmd = [B._hipcc(), "-shared", "-fPIC", f"--offload-arch={B.ARCH}"] + SAN + ["-o", lib] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return lib


def main():
    lib = build_sanitized(verbose="-v" in sys.argv)
    env = dict(os.environ, KDA_LIB=lib, LD_PRELOAD=asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",  # (the interpreter's own allocations)
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    test = os.path.join(B.ROOT, "tests", "test_abi.py")
    r = subprocess.run([sys.executable, "-m", "pytest", test, "-q", "-m", "not gpu", "-p", "no:cacheprovider"],
                       env=env, cwd=B.ROOT)
    print(f"sanitized library: {lib}; tests/test_abi.py exit status {r.returncode}")
    sys.exit(r.returncode)


if __name__ == "__main__":
    main()
