"""Build liblightning_attn.so for gfx950 with hipcc (in-tree).

    python -m long_context_decayed_amd.build        # or build() from Python

Objects go to _build/ at the repository root; the library lands next to this
file.  Always recompiles (it is the "does it build" check as well)."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblightning_attn.so")

SOURCES = ["la_abi.cpp", "la_state.hip", "la_output.hip", "la_decode.hip", "la_fused.hip"]

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    "--no-offload-compress",
    # Keep the compiler from forming packed-fp32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src):
    path = os.path.join(CSRC, src)
    obj = os.path.join(OUT_DIR, src + ".o")
    cmd = [_hipcc()] + HIP_FLAGS + ["-x", "hip", "-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
    warn = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    return obj, warn


def build(verbose=False):
    os.makedirs(OUT_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [r[0] for r in results]
    for _, warn in results:
        if warn and verbose:
            print("\n".join(warn), file=sys.stderr)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "--hip-link", "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
