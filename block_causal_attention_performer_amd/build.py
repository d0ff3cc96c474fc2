"""Build libbca.so (all HIP sources under csrc/) for gfx950 with hipcc.

Usage: python -m block_causal_attention_performer_amd.build [-D NAME=VALUE ...]
Objects go to _build/ next to this file; the library lands beside this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbca.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    """The library's HIP sources (every *.hip under csrc/)."""
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(defines=(), out: str = LIB, verbose: bool = False) -> str:
    srcs = sources()
    tag = "_".join(d.replace("=", "") for d in defines) or "default"
    objdir = os.path.join(HERE, "_build", tag)
    os.makedirs(objdir, exist_ok=True)
    # drop objects whose source is gone, so nothing links a deleted kernel
    keep = {os.path.basename(src) + ".o" for src in srcs}
    for o in glob.glob(os.path.join(objdir, "*.hip.o")):
        if os.path.basename(o) not in keep:
            os.remove(o)
    dflags = [f"-D{d}" for d in defines]
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [cc, *FLAGS, *dflags, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = out + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    defs = []
    args = sys.argv[1:]
    while args:
        a = args.pop(0)
        if a == "-D" and args:
            defs.append(args.pop(0))
        elif a.startswith("-D"):
            defs.append(a[2:])
        elif a == "-o" and args:
            globals()["LIB"] = args.pop(0)
    build(defs, out=LIB, verbose=True)
