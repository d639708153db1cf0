"""Build libpa.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Usage: ``python -m paged_kv_cache_hkv_amd.build`` (or ``build()`` from Python).
The library lands next to this file; the Python binding loads it from there.
Each source is compiled by hipcc on its own (in parallel), then linked.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpa.so")

SOURCES = [
    "pa_api.cpp",
    "pa_metadata.hip",
    "pa_cache_write.hip",
    "pa_blocks.hip",
    "pa_rope.hip",
    "pa_decode.hip",
    "pa_prefill.hip",
    "pa_noalloc.hip",
]

ARCH = "gfx950"

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    f"--offload-arch={ARCH}",
    # packed fp32 VALU ops stay off: hipcc must not form v_pk_{add,mul,fma}_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source additions.  pa_decode.hip: MFMA accumulators in ordinary VGPRs;
# with them in AGPRs the compiler copies every accumulator through VGPRs on
# each block (a segment's reset and the rescale touch them with VALU ops).
EXTRA_FLAGS = {
    "pa_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return exe


def build(verbose=False):
    """Compile every source and link libpa.so; raises on any compiler error."""
    os.makedirs(OBJDIR, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = ([hipcc()] + COMMON_FLAGS + EXTRA_FLAGS.get(src, []) + lang +
               ["-c", os.path.join(CSRC, src), "-o", obj])
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # the host pass does not know the packed-fp32 feature; that warning is harmless
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if p.returncode != 0:
            failed.append((src, "\n".join(lines)))
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        msg = "\n\n".join(f"[{s}]\n{t}" for s, t in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout.decode(errors="replace"))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
