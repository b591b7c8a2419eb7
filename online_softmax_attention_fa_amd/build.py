"""Build libfa.so (gfx950 only) in-tree with hipcc.

    python -m online_softmax_attention_fa_amd.build      # or __graft_entry__.build()

Each ``csrc/*.hip`` file is compiled to an object in parallel, then linked into
``online_softmax_attention_fa_amd/libfa.so``.  The build always recompiles.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 VALU ops are kept out of the generated code on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]


# Per-source extra hipcc flags, by file name (none at present).
FILE_FLAGS = {}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name; drop that noise
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, extra_flags=None, out: str = LIB) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    flags = COMMON_FLAGS + list(extra_flags or [])
    tmp = tempfile.mkdtemp(prefix="fa_build_")
    try:
        srcs = sources()
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]
        with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
            outs = list(ex.map(lambda so: _run([HIPCC, *flags, *FILE_FLAGS.get(os.path.basename(so[0]), []),
                                                "-c", so[0], "-o", so[1]]),
                               zip(srcs, objs)))
        if verbose:
            for o in outs:
                if o.strip():
                    print(o)
        tmp_lib = out + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib])
        os.replace(tmp_lib, out)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
