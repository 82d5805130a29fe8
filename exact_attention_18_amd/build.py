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
# The race-check variant: the same kernels with conservative synchronisation
# (ATTN_FORCE_SAFE); its outputs must equal libattn.so's bit for bit.
SAFE_LIB = os.path.join(PKG, "libattn_safe.so")
# The software-exp2 variant: 8 of every 32 exponentials of the d = 128 softmax
# on the FMA pipe (ATTN_EXP2_POLY=8); measured slower, so not the default.
EXP2POLY_LIB = os.path.join(PKG, "libattn_exp2poly.so")
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


def _compile(out: str, extra, verbose: bool) -> subprocess.Popen:
    tmp = out + ".tmp"
    cmd = [hipcc_path(), *compile_flags(extra), "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def _finish(out: str, proc: subprocess.Popen, verbose: bool) -> str:
    tmp = out + ".tmp"
    text, _ = proc.communicate()
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in text.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}) for {os.path.basename(out)}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    # Every symbol must resolve (e.g. host stubs of all kernel instantiations).
    try:
        ctypes.CDLL(tmp)
    except OSError as exc:
        os.remove(tmp)
        raise RuntimeError(f"built library does not load: {exc}") from exc
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, extra=(), variants: bool = True) -> str:
    """Compile libattn.so (and, with variants, libattn_safe.so and libattn_exp2poly.so).

    The compiles run side by side.  Returns libattn.so's path; raises on
    compiler failure.
    """
    jobs = [(LIB, _compile(LIB, extra, verbose))]
    if variants:
        jobs.append((SAFE_LIB, _compile(SAFE_LIB, (*extra, "-DATTN_FORCE_SAFE=1"), verbose)))
        jobs.append((EXP2POLY_LIB, _compile(EXP2POLY_LIB, (*extra, "-DATTN_EXP2_POLY=8"), verbose)))
    for out, proc in jobs:
        _finish(out, proc, verbose)
    return LIB


def build_variant(out: str, defines=(), verbose: bool = False) -> str:
    """Compile one library with extra -D defines (e.g. ATTN_EXP2_POLY=4) into `out`."""
    out = os.path.abspath(out)
    return _finish(out, _compile(out, tuple(f"-D{d}" for d in defines), verbose), verbose)


if __name__ == "__main__":
    import argparse

    ap = argparse.ArgumentParser(description="Build libattn.so and its variants for gfx950.")
    ap.add_argument("--define", action="append", default=[], metavar="NAME=VALUE",
                    help="build one variant with this preprocessor define (repeatable)")
    ap.add_argument("--out", default=None, help="output path of the variant (with --define)")
    a = ap.parse_args()
    if a.define:
        if not a.out:
            ap.error("--define needs --out")
        print(build_variant(a.out, a.define, verbose=True))
    else:
        print(build(verbose=True))
