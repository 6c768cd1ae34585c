"""Build libpkvattn.so for gfx950 with hipcc (in-tree, next to the Python binding).

Usage: python -m paged_kv_attention_causal_amd.csrc.build  (or call build()).
Each source compiles to its own object in parallel, then one shared link.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
OUT = os.path.join(PKG, "libpkvattn.so")
OBJDIR = os.path.join(PKG, "_build")
SOURCES = ["abi.cpp", "decode.hip", "prefill.hip", "mla.hip", "append.hip", "mla_proj.hip"]
ARCH = "gfx950"
# -packed-fp32-ops: no packed fp32 VALU ops in device code.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-munsafe-fp-atomics"]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def _compile(src, objdir=OBJDIR, defines=()):
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + FLAGS + [f"-D{d}" for d in defines] + ["-x", "hip", "-c",
                                                             os.path.join(HERE, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(verbose=False, out=OUT, defines=()):
    """Compile every source and link ``out``; ``defines`` are extra -D macros (tuning knobs)."""
    objdir = OBJDIR if out == OUT else out + ".objs"
    os.makedirs(objdir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        results = list(ex.map(lambda s: _compile(s, objdir, defines), SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for (o, err) in results:
            if err.strip():
                print(err, file=sys.stderr)
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
