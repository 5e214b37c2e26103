"""Build libdv.so (HIP for gfx950) in-tree with hipcc.

    python -m contextual_sparsity_decoding_amd.build [--changed]

Objects go to _build/ at the repository root; the library lands next to this
file, where the binding loads it.  build() compiles every source each time;
--changed recompiles only sources whose object is older than the source or
one of the headers it includes (from hipcc's dependency files).
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdv.so")
SYNTH_SRC = os.path.join(PKG, "synth_philox.c")
SYNTH_LIB = os.path.join(PKG, "libsynth.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function", "-Wno-unused-result",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _obj(src: str) -> str:
    return os.path.join(OBJDIR, os.path.basename(src) + ".o")


def _stale(src: str) -> bool:
    """True when the object is missing or older than anything it was built from."""
    obj, dep = _obj(src), _obj(src) + ".d"
    if not (os.path.exists(obj) and os.path.exists(dep)):
        return True
    t = os.path.getmtime(obj)
    with open(dep) as f:
        names = f.read().replace("\\\n", " ").split()
    for n in names[1:]:
        if n.endswith(":"):
            continue
        if not os.path.exists(n) or os.path.getmtime(n) > t:
            return True
    return False


def _compile(src: str) -> str:
    obj = _obj(src)
    cmd = [hipcc(), *FLAGS, "-MMD", "-MF", obj + ".d", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and "ignoring feature" not in l)
    if warn.strip():
        sys.stderr.write(warn + "\n")
    return obj


def build_synth(verbose: bool = True) -> str:
    """The host side of the seeded input generator (plain C, gcc, OpenMP)."""
    tmp = SYNTH_LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-Wall", SYNTH_SRC, "-o", tmp, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed on {SYNTH_SRC}:\n{r.stderr}")
    os.replace(tmp, SYNTH_LIB)
    if verbose:
        print(f"built {SYNTH_LIB}")
    return SYNTH_LIB


def build(verbose: bool = True, changed_only: bool = False) -> str:
    if not changed_only or not os.path.exists(SYNTH_LIB) or os.path.getmtime(SYNTH_LIB) < os.path.getmtime(SYNTH_SRC):
        build_synth(verbose)
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    todo = [s for s in srcs if _stale(s)] if changed_only else srcs
    # the slowest sources first, so the pool's last jobs are short ones
    todo.sort(key=lambda s: -os.path.getsize(s) - (1 << 20) * ("qkv" in s))
    if todo:
        with ThreadPoolExecutor(min(8, len(todo))) as ex:
            list(ex.map(_compile, todo))
    objs = [_obj(s) for s in srcs]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(changed_only="--changed" in sys.argv[1:])
