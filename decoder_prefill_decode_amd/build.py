"""Builds libvlm.so (the C-ABI library with every gfx950 kernel) in-tree.

python -m decoder_prefill_decode_amd.build  [-j N]
"""
import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libvlm.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["api.hip", "k_misc.hip", "k_gemm.hip", "k_gemv.hip", "k_attn.hip", "k_sample.hip", "k_gemm_small.hip"]
ARCH = "gfx950"

# Packed-fp32 instructions stay off: the compiler would otherwise form
# v_pk_* fp32 ops from plain float code.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc():
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l]
    return p.returncode, "\n".join(lines)


def build(jobs: int = 8, verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libvlm.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()

    def one(src):
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        rc, out = _run([cc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        return src, obj, rc, out

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        results = list(ex.map(one, SOURCES))
    errs = [(s, o) for s, _, rc, o in results if rc != 0]
    for s, _, rc, o in results:
        if (verbose or rc) and o.strip():
            print(f"--- {s}\n{o}", file=sys.stderr)
    if errs:
        raise RuntimeError("HIP compilation failed: " + ", ".join(s for s, _ in errs))
    tmp = OUT + ".tmp"
    rc, out = _run([cc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *[o for _, o, _, _ in results]])
    if rc != 0:
        print(out, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=8)
    ap.add_argument("-v", action="store_true")
    a = ap.parse_args()
    print(build(a.j, a.v))
