"""Builds libmoe.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run as ``python -m quantized_expert_ffn_top_amd._build``; ``__graft_entry__.build``
calls :func:`build`.  Every translation unit is compiled in parallel, then
linked into ``quantized_expert_ffn_top_amd/libmoe.so`` (replaced atomically).
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe.so")
SOURCES = ["moe_api.hip", "moe_kernels_small.hip", "moe_kernels_decode.hip",
           "moe_kernels_gemm.hip", "moe_kernels_dense.hip"]
LINK = []

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         # packed fp32 instructions are kept out of the generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), out))
    return out


def build(verbose=False):
    tmp = tempfile.mkdtemp(prefix="moe_build_")
    try:
        objs = []
        cmds = []
        for s in SOURCES:
            o = os.path.join(tmp, s.replace(".hip", ".o"))
            objs.append(o)
            cmds.append([HIPCC] + FLAGS + ["-c", os.path.join(CSRC, s), "-o", o])
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            for out in ex.map(_run, cmds):
                if verbose and out.strip():
                    print(out)
        tmp_lib = os.path.join(tmp, "libmoe.so")
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_lib] + objs + LINK)
        shutil.copyfile(tmp_lib, LIB + ".tmp")
        os.replace(LIB + ".tmp", LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
