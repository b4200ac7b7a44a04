"""Host-side sanitizer run: builds the oracle, the host input generator and
the library (its host code: argument checks, workspace carving, tier
bookkeeping) with AddressSanitizer and UndefinedBehaviorSanitizer, then runs
the CPU test suite (pytest -m "not gpu") on those builds.

Device code is never sanitized: the library's hipcc line passes each
-fsanitize= option to the host compilation only (-Xarch_host).  All three
builds use the same clang (ROCm's), so one sanitizer runtime serves the
process; it is preloaded into the Python interpreter.

    python tests/sanitize_host.py            # build, then run the CPU suite
Exit status: pytest's.  The builds go to _build/asan/ (not tracked).
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "asan")
CLANG = "/opt/rocm/llvm/bin/clang"
HIPCC = "/opt/rocm/bin/hipcc"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
       "-g", "-O1", "-shared-libsan"]


def run(cmd):
    print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build():
    os.makedirs(OUT, exist_ok=True)
    run([CLANG, "-std=c11", *SAN, "-ffp-contract=off", "-fPIC", "-shared", "-Wall", "-o",
         os.path.join(OUT, "libmoe_ref.so"), os.path.join(ROOT, "oracle", "moe_ref.c"), "-lm"])
    run([CLANG, "-std=c11", *SAN, "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-Wall",
         "-o", os.path.join(OUT, "libsynth_host.so"), os.path.join(ROOT, "synth", "synth_host.c"),
         "-lm"])
    sys.path.insert(0, ROOT)
    from int4_expert_gemv_moe_amd import build as lib_build
    host_san = []
    for f in SAN:
        host_san += ["-Xarch_host", f]
    objs = []
    for src in lib_build.SOURCES:
        obj = os.path.join(OUT, src.replace(".hip", ".o"))
        run([HIPCC, *lib_build.FLAGS, *host_san, "-c", os.path.join(lib_build.CSRC, src), "-o", obj])
        objs.append(obj)
    run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address,undefined",
         "-Xarch_host", "-shared-libsan", "-o", os.path.join(OUT, "libmoe_i4.so"), *objs])


def main():
    build()
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rt:
        raise SystemExit("clang's AddressSanitizer runtime is not installed")
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt[0],
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               MOE_REF_LIB=os.path.join(OUT, "libmoe_ref.so"),
               SYNTH_HOST_LIB=os.path.join(OUT, "libsynth_host.so"),
               MOE_I4_LIB=os.path.join(OUT, "libmoe_i4.so"))
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-x", "-m", "not gpu",
           "-p", "no:cacheprovider"]
    print(" ".join(cmd), flush=True)
    sys.exit(subprocess.run(cmd, env=env, cwd=ROOT).returncode)


if __name__ == "__main__":
    main()
