"""Build libmla.so (gfx950) in-tree with hipcc.

    python -m sparse_mla_attention_decode_amd.build

Compiles every .hip source under csrc/ into one shared library next to this
file.  Packed-fp32 VALU instructions are disabled for device code.
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
LIB = os.path.join(PKG, "libmla.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmla)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def compile_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", f"-I{INCLUDE}", f"-I{CSRC}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-Wno-unused-parameter"]


def build(verbose: bool = False, extra=()) -> str:
    out_tmp = LIB + ".tmp"
    cmd = [hipcc(), *compile_flags(), "-shared", "-o", out_tmp, *sources(), *extra]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is expected
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops" not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("libmla build failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(out_tmp, LIB)
    return LIB


def sanitizer_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (raises if absent)."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the AddressSanitizer runtime was not found")
    return path


def build_sanitized(out: str) -> str:
    """The same library with its host code under AddressSanitizer and
    UndefinedBehaviorSanitizer (device code is built as usual: every
    sanitizer flag applies to the host pass only).  For host-side tests run
    with the runtime preloaded (sanitizer_runtime)."""
    host = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
              "-fno-omit-frame-pointer"):
        host += ["-Xarch_host", f]
    flags = [f for f in compile_flags() if f != "-O3"]
    cmd = [hipcc(), "-O1", "-g", *flags, *host, "-shared-libsan", "-shared", "-o", out, *sources()]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("sanitized libmla build failed:\n" + res.stderr[-4000:])
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
