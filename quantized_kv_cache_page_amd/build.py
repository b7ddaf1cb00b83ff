"""Build libskvd.so in-tree with hipcc for gfx950.

    python -m quantized_kv_cache_page_amd.build

Every HIP translation unit is compiled with packed-FP32 instructions disabled (the compiler
otherwise forms v_pk_* f32 operations by itself).
"""
from __future__ import annotations

import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libskvd.so")
PARTIAL = [f"partial_{d}_{f}.hip" for d in (128, 256, 512)
           for f in ("f16", "i8", "f8", "q4")] + ["partial_192_f16.hip", "partial_192_f8.hip"]
SOURCES = ["api.cpp", "plan.cpp", "kernels.hip", *PARTIAL, "append.hip", "prefill.hip",
           "cascade.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = True, out: str = LIB) -> str:
    """Compile the sources (in parallel) and link libskvd.so. Returns the library path."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
              "-Wno-unused-result", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", os.path.join(ROOT, "include")]
    procs, objs = [], []
    t0 = time.time()
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        lang = ["-x", "hip"] if src.endswith((".hip", ".cpp")) else []
        cmd = [hipcc(), *common, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = False
    for src, p in procs:
        out_txt = p.communicate()[0].decode(errors="replace")
        noise = "is not a recognized feature for this target"
        lines = [ln for ln in out_txt.splitlines() if noise not in ln]
        if p.returncode != 0:
            failed = True
            sys.stderr.write(f"hipcc failed on {src}:\n" + "\n".join(lines) + "\n")
        elif verbose and lines:
            sys.stderr.write("\n".join(lines) + "\n")
    if failed:
        raise RuntimeError("libskvd build failed")
    tmp = out + ".tmp"
    subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, out)
    if verbose:
        sys.stderr.write(f"built {out} in {time.time() - t0:.1f}s\n")
    return out


if __name__ == "__main__":
    build()
