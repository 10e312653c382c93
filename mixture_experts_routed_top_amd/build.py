"""Build the HIP library libmoe_mi355x.so in-tree for gfx950.

Every source under csrc/ is compiled to an object with hipcc (in parallel)
and linked into mixture_experts_routed_top_amd/libmoe_mi355x.so. Always
recompiles: it is the "does it build" check as well as the build.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_mi355x.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 arithmetic is kept off: the compiler then never forms
    # v_pk_{add,mul,fma}_f32 from ordinary float code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


PROBES = os.path.join(HERE, "probes")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def build_probes(verbose: bool = False):
    """The matrix-core measurement probes (probes/*.hip), each a small
    stand-alone executable next to its source."""
    out = []
    for f in sorted(os.listdir(PROBES)):
        if not f.endswith(".hip"):
            continue
        src, exe = os.path.join(PROBES, f), os.path.join(PROBES, f[:-4])
        r = subprocess.run([HIPCC, *FLAGS, src, "-o", exe], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        out.append(exe)
    if verbose:
        print(f"built {len(out)} probe(s) in {PROBES}")
    return out


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    build_probes(verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
