"""Run the host-side tests under AddressSanitizer + UndefinedBehaviorSanitizer
(CPU only; no GPU code is instrumented).

  1. The C oracle built with gcc -fsanitize=address,undefined, and the oracle
     pins (tests/test_oracle_pins.py) run against it, with gcc's ASan runtime
     preloaded into the interpreter.
  2. libkvq built with the sanitizers on its host code only (each hipcc line
     puts -Xarch_host before every -fsanitize=; device code is built as
     usual), and the C-ABI tests (tests/test_abi.py: argument checks, plans,
     workspace sizes, the stale-build check) run against it, with clang's ASan
     runtime preloaded.

The two runtimes cannot share a process, so each suite runs in its own.  Leak
detection is off (the interpreter keeps its allocations until exit); any
other report fails the run.  Usage: python tests/run_sanitizers.py
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
OUT = os.path.join(ROOT, "_build", "sanitize")

ENV_ASAN = "detect_leaks=0:halt_on_error=1:abort_on_error=0:detect_odr_violation=0"
ENV_UBSAN = "halt_on_error=1:print_stacktrace=1"


def run(cmd, env=None):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, env=env)


def build_oracle():
    src = os.path.join(ROOT, "oracle", "kvq_oracle.c")
    out = os.path.join(OUT, "libkvq_oracle_san.so")
    run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared", "-fPIC",
         "-o", out, src, "-lm"])
    return out


def build_library():
    from bit_quantized_kv_rotate_amd import _build as B
    objs = []
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-Xarch_host", "-g"]
    for name, extra in B.SOURCES.items():
        obj = os.path.join(OUT, name + ".o")
        run([B.HIPCC] + B.COMMON + extra + san + ["-c", os.path.join(B.CSRC, name), "-o", obj])
        objs.append(obj)
    out = os.path.join(OUT, "libkvq_san.so")
    run([B.HIPCC, "--offload-arch=" + B.ARCH, "-shared", "-fPIC", "-shared-libsan",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-o", out] + objs)
    with open(out + ".srchash", "w") as f:
        f.write(B.source_hash() + "\n")
    return out


def instrumented(lib):
    """The build calls into the ASan runtime (its host code is instrumented)."""
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True,
                          check=True).stdout
    if "__asan_report" not in syms or "__ubsan_handle" not in syms:
        raise SystemExit("%s is not instrumented" % lib)


def main():
    os.makedirs(OUT, exist_ok=True)
    # 1. oracle pins against the instrumented oracle
    orc = build_oracle()
    instrumented(orc)
    gcc_asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                              check=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=gcc_asan, ASAN_OPTIONS=ENV_ASAN, UBSAN_OPTIONS=ENV_UBSAN,
               KVQ_ORACLE_LIB=orc)
    run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", os.path.join(ROOT, "tests",
                                                                                     "test_oracle_pins.py")], env)
    # 2. C-ABI tests against libkvq with instrumented host code
    lib = build_library()
    instrumented(lib)
    rt = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        raise SystemExit("clang ASan runtime not found")
    env = dict(os.environ, LD_PRELOAD=rt[-1], ASAN_OPTIONS=ENV_ASAN, UBSAN_OPTIONS=ENV_UBSAN, KVQ_LIBRARY=lib)
    run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", os.path.join(ROOT, "tests",
                                                                                     "test_abi.py")], env)
    print("sanitizer runs clean")


if __name__ == "__main__":
    main()
