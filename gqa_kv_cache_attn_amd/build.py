"""Build libgqa_decode.so in-tree with hipcc for gfx950.

    python -m gqa_kv_cache_attn_amd.build

Every HIP translation unit is compiled with packed-fp32 ops disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops); hipcc's host pass warns
that it does not know that feature, which is harmless.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libgqa_decode.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["gqa_kernels.hip", "gqa_paged.hip", "gqa_api.hip"]
ARCH = "gfx950"


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (looked at $HIPCC, /opt/rocm/bin/hipcc, PATH)")


def compile_command(out_path: str, sources=SOURCES) -> list:
    return [
        hipcc_path(), f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-shared",
        "-fvisibility=hidden", "-Wall", "-Wno-unused-command-line-argument",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        *[os.path.join(CSRC, s) for s in sources],
        "-o", out_path,
    ]


def _compile(sources, out_path, verbose):
    tmp = out_path + f".tmp{os.getpid()}"
    cmd = compile_command(tmp, sources)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.unlink(tmp)
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    noise = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)
    os.replace(tmp, out_path)


def build(verbose: bool = False) -> str:
    """Compile the library (always; no staleness shortcut); return its path."""
    _compile(SOURCES, LIB_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
