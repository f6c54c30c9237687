"""Builds libcoli_moe.so in place with hipcc for gfx950 (every HIP source
plus the C ABI). Run as a script or through __graft_entry__.build().

`python -m int4_quantized_expert_sigmoid_amd.build --trace` builds the
profiling variant instead, _trace/libcoli_moe.so: the same sources with
COLI_TRACE defined, whose decode kernels stamp every workgroup's phases into
a buffer the caller installs (see trace_decode.py)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcoli_moe.so")
TRACE_LIB = os.path.join(HERE, "_trace", "libcoli_moe.so")
SOURCES = ["abi.cpp", "kernels_quant.hip", "kernels_route.hip", "kernels_gemv.hip", "kernels_grouped.hip",
           "kernels_combine.hip",
           "kernels_decode.hip", "kernels_dense.hip"]
# The grouped MFMA kernels read every MFMA result with VALU instructions; in
# VGPR form the accumulator copies (one per result) disappear.
SOURCE_FLAGS = {"kernels_grouped.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "kernels_route.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fno-fast-math", "-ffp-contract=fast-honor-pragmas", "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False, jobs: int = 8, trace: bool = False) -> str:
    objdir = os.path.join(HERE, "_build_trace" if trace else "_build")
    out = TRACE_LIB if trace else LIB
    defines = ["-DCOLI_TRACE"] if trace else []
    os.makedirs(objdir, exist_ok=True)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = ["hipcc", *FLAGS, *SOURCE_FLAGS.get(src, []), *defines, "-c", *lang, os.path.join(CSRC, src), "-o", obj]
        cmd = [c for c in cmd if c != "-shared"]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        _, err = p.communicate()
        msgs = [l for l in err.splitlines() if "packed-fp32-ops" not in l]
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write("\n".join(msgs) + "\n")
        elif verbose and msgs:
            sys.stderr.write("\n".join(msgs) + "\n")
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    link = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    return out


if __name__ == "__main__":
    build(verbose=True, trace="--trace" in sys.argv[1:])
