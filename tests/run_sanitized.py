"""Host-sanitizer run of the CPU test suite (AddressSanitizer + UBSan).

Builds, with ROCm's clang, so that the whole process has one sanitizer
runtime:
  oracle/_asan/liboracle.so, liboracle_omp.so   the oracle, both builds
  synth/_asan/libsynth.so                        the input generator
  int4_quantized_expert_sigmoid_amd/_asan/libcoli_moe.so
      the library with its host code instrumented (argument checks, host
      packers, workspace layout); its device code is built as usual and
      is not instrumented. This is a CPU run: no test here launches a
      kernel.
Then it runs `pytest -m "not gpu"` in a child process with the runtime
preloaded and COLI_LIB_VARIANT=asan, which makes the three loaders pick these
builds. Any AddressSanitizer or UBSan report ends the run with a nonzero
status.

    python tests/run_sanitized.py [extra pytest arguments]
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
CLANG = "/opt/rocm/llvm/bin/clang"
LLVM_LIB = "/opt/rocm/llvm/lib"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


def run(cmd):
    print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build_oracle():
    d = os.path.join(ROOT, "oracle")
    out = os.path.join(d, "_asan")
    os.makedirs(out, exist_ok=True)
    base = [CLANG, *SAN, "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-shared-libsan",
            "-Wall", "-Wno-unused-parameter", os.path.join(d, "oracle.c"), "-lm"]
    run(base + ["-Wno-unknown-pragmas", "-o", os.path.join(out, "liboracle.so")])
    run(base + ["-fopenmp", f"-Wl,-rpath,{LLVM_LIB}", "-o", os.path.join(out, "liboracle_omp.so")])


def build_synth():
    d = os.path.join(ROOT, "synth")
    out = os.path.join(d, "_asan")
    os.makedirs(out, exist_ok=True)
    run([CLANG, *SAN, "-std=c99", "-fopenmp", f"-Wl,-rpath,{LLVM_LIB}", "-fPIC", "-shared", "-shared-libsan",
         os.path.join(d, "synth.c"), "-o", os.path.join(out, "libsynth.so"), "-lm"])


def build_library():
    from int4_quantized_expert_sigmoid_amd import build as B
    out = os.path.join(B.HERE, "_asan")
    objdir = os.path.join(B.HERE, "_build_asan")
    os.makedirs(out, exist_ok=True)
    os.makedirs(objdir, exist_ok=True)
    # host-side instrumentation only (each sanitizer flag applies to the host pass)
    host = []
    for f in SAN:
        host += ["-Xarch_host", f]
    objs = []
    for src in B.SOURCES:
        obj = os.path.join(objdir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        flags = [f for f in B.FLAGS if f != "-shared"]
        run(["hipcc", *flags, *B.SOURCE_FLAGS.get(src, []), *host, "-c", *lang, os.path.join(B.CSRC, src), "-o", obj])
        objs.append(obj)
    run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address,undefined",
         "-Xarch_host", "-shared-libsan", *objs, "-o", os.path.join(out, "libcoli_moe.so")])


def check_instrumented(paths):
    """Each built library must call into the sanitizer runtimes."""
    for p in paths:
        syms = subprocess.run(["nm", "-D", "--undefined-only", p], check=True, capture_output=True, text=True).stdout
        if "__asan_" not in syms or "__ubsan_handle_" not in syms:
            raise SystemExit(f"{p} is not instrumented")


def main(argv):
    build_oracle()
    build_synth()
    build_library()
    check_instrumented([os.path.join(ROOT, "oracle", "_asan", "liboracle.so"),
                        os.path.join(ROOT, "oracle", "_asan", "liboracle_omp.so"),
                        os.path.join(ROOT, "synth", "_asan", "libsynth.so"),
                        os.path.join(ROOT, "int4_quantized_expert_sigmoid_amd", "_asan", "libcoli_moe.so")])
    runtime = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], check=True,
                             capture_output=True, text=True).stdout.strip()
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime, COLI_LIB_VARIANT="asan",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               LD_LIBRARY_PATH=LLVM_LIB + (":" + env["LD_LIBRARY_PATH"] if env.get("LD_LIBRARY_PATH") else ""))
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m", "not gpu", "-q", "-p", "no:cacheprovider",
           *argv]
    print("running the CPU suite under AddressSanitizer + UBSan:", " ".join(cmd), flush=True)
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
