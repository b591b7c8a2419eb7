"""Build libfa.so (gfx950 only) in-tree with hipcc.

    python -m online_softmax_attention_fa_amd.build      # or __graft_entry__.build()

Each ``csrc/*.hip`` file is compiled to an object in parallel, then linked into
``online_softmax_attention_fa_amd/libfa.so``.  The same run also links the LDS-poison debug
build, ``libfa_poison.so``: the forward kernels recompiled with ``-DFA_LDS_POISON`` (every
K/V tile buffer filled with NaN before its copy), which a subset of the GPU parity tests
runs.  The build always recompiles.
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
POISON_LIB = os.path.join(PKG, "libfa_poison.so")
# the source whose kernels the poison build changes
POISON_SOURCE = "fa_fwd_kernel.hip"

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


def build(verbose: bool = False, extra_flags=None, out: str = LIB, link_flags=None, poison_out=None) -> str:
    """Compile every source and link ``out``; with ``poison_out``, also compile the forward
    kernels with -DFA_LDS_POISON and link that debug build from the same objects."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    flags = COMMON_FLAGS + list(extra_flags or [])
    tmp = tempfile.mkdtemp(prefix="fa_build_")
    try:
        srcs = sources()
        jobs = [(s, os.path.join(tmp, os.path.basename(s) + ".o"), []) for s in srcs]
        poison_src = os.path.join(CSRC, POISON_SOURCE)
        if poison_out:
            jobs.append((poison_src, os.path.join(tmp, "poison_" + POISON_SOURCE + ".o"), ["-DFA_LDS_POISON"]))
        with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
            outs = list(ex.map(lambda j: _run([HIPCC, *flags, *FILE_FLAGS.get(os.path.basename(j[0]), []), *j[2],
                                               "-c", j[0], "-o", j[1]]),
                               jobs))
        if verbose:
            for o in outs:
                if o.strip():
                    print(o)
        objs = [o for s, o, x in jobs if not x]
        targets = [(out, objs)]
        if poison_out:
            targets.append((poison_out, [o if s != poison_src else jobs[-1][1] for s, o, x in jobs if not x]))
        for lib, lib_objs in targets:
            tmp_lib = lib + ".tmp"
            _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *list(link_flags or []), *lib_objs,
                  "-o", tmp_lib])
            os.replace(tmp_lib, lib)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, poison_out=POISON_LIB))
