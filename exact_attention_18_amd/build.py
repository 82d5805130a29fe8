"""Ahead-of-time build of libattn.so for gfx950 with hipcc.

Compiles every HIP source of the library into one shared object next to this
file.  It always compiles (no staleness check): callers that only want to load
an existing build use ``exact_attention_18_amd.attn``.

Flags: -O3 for gfx950 only; packed-FP32 VALU instructions are disabled with
``-Xclang -target-feature -Xclang -packed-fp32-ops`` (the host pass prints a
harmless notice that it does not know this feature).
"""

from __future__ import annotations

import ctypes
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
SOURCES = [os.path.join(PKG, "csrc", n) for n in ("attn_fwd.hip", "attn_bwd.hip", "mfma_probe.hip")]
LIB = os.path.join(PKG, "libattn.so")
ARCH = "gfx950"


def hipcc_path() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (expected a ROCm installation under /opt/rocm)")


def compile_flags(extra=()):
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        *extra,
    ]


def build(verbose: bool = False, extra=()) -> str:
    """Compile libattn.so; returns its path.  Raises on compiler failure."""
    tmp = LIB + ".tmp"
    cmd = [hipcc_path(), *compile_flags(extra), "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    # Every symbol must resolve (e.g. host stubs of all kernel instantiations).
    try:
        ctypes.CDLL(tmp)
    except OSError as exc:
        os.remove(tmp)
        raise RuntimeError(f"built library does not load: {exc}") from exc
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
