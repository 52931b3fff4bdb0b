"""Build the HIP library libfa.so in-tree for gfx950 with hipcc.

Every call recompiles (the build is the "does it compile" check); objects are
compiled in parallel and linked into exact_attention_03_amd/libfa.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_paged.hip", "fa_quest.hip", "fa_noalloc.hip", "fa_bwd_fused.hip"]
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler away from packed fp32 VALU forms
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")


def _quiet(text: str) -> str:
    # The host pass does not know the packed-fp32 target feature; that warning is noise.
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    cc = hipcc()
    flags = COMMON + list(extra_flags or [])
    with tempfile.TemporaryDirectory(prefix="fa_build_") as tmp:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmd = [cc, *flags, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        errors = []
        for src, p in procs:
            out, _ = p.communicate()
            out = _quiet(out)
            if p.returncode != 0:
                errors.append(f"--- {src} ---\n{out}")
            elif verbose and out.strip():
                print(out)
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
        tmp_lib = LIB + ".tmp"
        cmd = [cc, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp_lib]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + _quiet(r.stdout))
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
