"""Build libgtms.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

The kernel launchers are compiled once per operation (forward, backward) and mask kind
(tril, band, explicit mask) from launch_kind.hip, in parallel with the fused attention
launcher (launch_attention.hip) and the host logic (gtms_api.hip); the objects are then
linked into one shared library.
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
LIB = os.path.join(PKG, "libgtms.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC",
    # keep the compiler from emitting packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

# (source, extra defines) of every object in the library
UNITS = [("gtms_api.hip", []), ("launch_attention.hip", [])] + [
    ("launch_kind.hip", [f"-DGTMS_OP={op}", f"-DGTMS_MK={mk}"])
    for op in (0, 1) for mk in (0, 1, 2)
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmds):
    """Runs the commands in parallel; raises with the first failure's output."""
    procs = [subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
             for c in cmds]
    outs = [p.communicate() for p in procs]
    for c, p, (o, e) in zip(cmds, procs, outs):
        if p.returncode != 0:
            sys.stderr.write(o + e)
            raise RuntimeError(f"hipcc failed ({p.returncode}): {' '.join(c)}")
    return outs


def build(extra_flags=(), out: str = LIB, quiet: bool = True) -> str:
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="gtms_build_") as tmp:
        objs, cmds = [], []
        for i, (src, defs) in enumerate(UNITS):
            obj = os.path.join(tmp, f"unit{i}.o")
            objs.append(obj)
            cmds.append([cc, *HIPCC_FLAGS, *extra_flags, *defs, f"-I{INCLUDE}", f"-I{CSRC}",
                         "-c", os.path.join(CSRC, src), "-o", obj])
        outs = _run(cmds)
        outs += _run([[cc, "--offload-arch=gfx950", "-fPIC", "-shared", *objs,
                       "-o", out + ".tmp"]])
    if not quiet:
        for _, e in outs:
            sys.stderr.write(e)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(quiet=False))
