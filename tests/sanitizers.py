"""Host-side AddressSanitizer / UndefinedBehaviorSanitizer builds, CPU only.

- liblinattn.so with the sanitizers on its host code (`-Xarch_host` before
  each -fsanitize, so the GPU code is built as usual), linked against the
  clang runtime: the C ABI's argument checks, segmentation plans and
  workspace formulas run instrumented.
- liboracle.so (oracle.c) built by gcc with -fsanitize=address,undefined.

Each runs pytest on the CPU tests that exercise it, in a subprocess with the
matching runtime preloaded (the two runtimes cannot share a process):
LINATTN_LIBRARY / LINATTN_ORACLE_LIB point the binding and the oracle at the
instrumented builds.  `python tests/sanitizers.py` builds and runs both.
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "san")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-g",
            "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def gcc_runtimes():
    out = []
    for lib in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["gcc", f"-print-file-name={lib}"], capture_output=True, text=True).stdout.strip()
        out.append(p)
    return out


def build_library():
    os.makedirs(OUT, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(ROOT, "kernelized_linear_attention_amd", "csrc", "*.hip")))
    flags = ["--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form", "-I",
             os.path.join(ROOT, "include"), *SAN_HOST]

    def one(src):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        r = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-3000:]}")
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(one, srcs))
    lib = os.path.join(OUT, "liblinattn.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host",
                    "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", *objs, "-o", lib],
                   check=True, capture_output=True)
    return lib


def build_oracle():
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "liboracle.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                    "-fno-fast-math", "-ffp-contract=off", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", lib, "-lm"], check=True)
    return lib


def run_pytest(test_files, preload, extra_env, timeout=900):
    env = dict(os.environ, **SAN_ENV, **extra_env, LD_PRELOAD=" ".join(preload))
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           "-m", "not gpu", *test_files], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=timeout)


def run_library_checks(lib):
    return run_pytest(["tests/test_abi.py"], [clang_asan_runtime()], {"LINATTN_LIBRARY": lib})


def run_oracle_checks(lib):
    return run_pytest(["tests/test_oracle_pins.py"], gcc_runtimes(), {"LINATTN_ORACLE_LIB": lib})


if __name__ == "__main__":
    ok = True
    for name, build, run in (("library host code", build_library, run_library_checks),
                             ("oracle", build_oracle, run_oracle_checks)):
        r = run(build())
        print(f"== {name} under ASan + UBSan: rc={r.returncode}")
        print(r.stdout[-1500:], r.stderr[-1500:])
        ok = ok and r.returncode == 0
    sys.exit(0 if ok else 1)
