"""Build the HIP library libcsmla.so in-tree for gfx950 (MI355X).

The library is the product's only compute path: the C ABIs in include/csmla.h
(attention) and include/csmla_indexer.h (indexer top-k), implemented by
csrc/csmla_host.cpp and csrc/csmla_indexer_host.cpp (validation, planners,
launches) and csrc/csmla_kernels.hip / csrc/csmla_indexer_kernels.hip.  Built with hipcc; no JIT cache.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcsmla.so")
BUILD = os.path.join(HERE, "_build")
ARCH = os.environ.get("CSMLA_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# gfx950 code is built without packed-fp32 instructions (v_pk_*_f32).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and "unknown-feature" not in l
                    and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}")
    if verbose and out:
        print(out)


def build(verbose: bool = False, save_temps: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    common = ["-std=c++17", "-O3", "-fPIC", "-Wall", "-Wno-unused-function"]
    objs = []
    for src in ("csmla_host.cpp", "csmla_indexer_host.cpp"):
        o = os.path.join(BUILD, src.replace(".cpp", ".o"))
        _run([HIPCC, *common, "-x", "c++", "-c", os.path.join(CSRC, src), "-o", o], verbose)
        objs.append(o)
    for src in ("csmla_kernels.hip", "csmla_indexer_kernels.hip"):
        o = os.path.join(BUILD, src.replace(".hip", ".o"))
        kcmd = [HIPCC, *common, f"--offload-arch={ARCH}", *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", o]
        if save_temps:
            kcmd += ["-save-temps=obj"]
        _run(kcmd, verbose)
        objs.append(o)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, save_temps="--save-temps" in sys.argv))
