"""Sanitizer runs on the CPU (AddressSanitizer + UndefinedBehaviorSanitizer), host code only.

1. The oracle (oracle/oracle.c) built by gcc with -fsanitize=address,undefined; the oracle pins
   (tests/test_oracle_pins.py) run against that build in a subprocess.
2. libfuse with its host code -- argument validation, launch plans, dispatch -- built by hipcc
   with the same sanitizers applied to the host pass only (the gfx950 code is compiled as
   usual); the C-ABI tests (tests/test_abi.py) run against it in a subprocess.  There is no GPU
   here: validation answers every call those tests make before anything is launched.
3. Controls: a one-element heap overflow and a signed integer overflow in throwaway C files,
   built with each sanitizer, must abort, so that a green run means the sanitizers were active.

Undefined behaviour is fatal (-fno-sanitize-recover); leak checking is off (the Python
interpreter itself is not leak-clean).  The sanitized libfuse is cached under _build/asan and
rebuilt only when a source is newer.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "memory_bound_amd", "csrc")
ASAN_DIR = os.path.join(ROOT, "_build", "asan")
HIPCC = "/opt/rocm/bin/hipcc"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}
GCC_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
# host pass only: every sanitizer flag behind -Xarch_host
HIP_HOST_SAN = [f for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
                               "-fno-omit-frame-pointer") for f in ("-Xarch_host", flag)]


def _gcc_runtime():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    rt = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("gcc has no AddressSanitizer runtime")
    return gcc, rt


def _clang_runtime():
    rts = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rts or not os.path.exists(HIPCC):
        pytest.skip("no hipcc / clang AddressSanitizer runtime")
    return rts[-1]


def _run_python(code, env_extra, timeout=900):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


@pytest.mark.parametrize("flag,body,expect", [
    ("-fsanitize=address", "volatile int *p = malloc(4 * sizeof(int)); int v = p[argc + 3]; free((void *)p);",
     "heap-buffer-overflow"),
    ("-fsanitize=undefined", "volatile int big = 2147483600; int v = big + argc * 100;",
     "signed integer overflow"),
])
def test_sanitizer_controls_fire(tmp_path, flag, body, expect):
    gcc, rt = _gcc_runtime()
    src = tmp_path / "bad.c"
    src.write_text("#include <stdlib.h>\nint main(int argc, char **argv) {\n  (void)argv;\n  " + body +
                   "\n  return v == 12345;\n}\n")
    exe = tmp_path / "bad"
    subprocess.run([gcc, "-O1", "-g", flag, "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=dict(os.environ, **SAN_ENV), timeout=60)
    assert r.returncode != 0 and expect in r.stderr, r.stderr[-2000:]


def test_oracle_pins_under_asan_ubsan(tmp_path):
    gcc, rt = _gcc_runtime()
    lib = tmp_path / "liboracle_san.so"
    subprocess.run([gcc, "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-fno-fast-math", *GCC_SAN, "-o", str(lib), os.path.join(ROOT, "oracle", "oracle.c"), "-lm"],
                   check=True)
    code = ("import sys, pytest; sys.exit(pytest.main(['-x', '-q', '-p', 'no:cacheprovider', "
            "'tests/test_oracle_pins.py']))")
    r = _run_python(code, {"ORACLE_LIB": str(lib), "LD_PRELOAD": rt})
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout


def _sanitized_libfuse():
    lib = os.path.join(ASAN_DIR, "libfuse.so")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.hpp")) +
                  [os.path.join(ROOT, "include", "libfuse.h")])
    if os.path.exists(lib) and os.path.getmtime(lib) >= max(os.path.getmtime(s) for s in srcs):
        return lib
    os.makedirs(ASAN_DIR, exist_ok=True)
    flags = ["-O1", "-g", "--offload-arch=gfx950", "-std=c++20", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
             *HIP_HOST_SAN, "-I", os.path.join(ROOT, "include")]
    procs, objs = [], []
    for s in srcs:
        if not s.endswith(".hip"):
            continue
        o = os.path.join(ASAN_DIR, os.path.basename(s)[:-4] + ".o")
        objs.append(o)
        procs.append(subprocess.Popen([HIPCC, *flags, "-c", s, "-o", o], stdout=subprocess.PIPE,
                                      stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out, _ = p.communicate(timeout=1200)
        assert p.returncode == 0, out[-4000:]
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-shared-libsan", "-o", lib + ".tmp", *objs],
                   check=True)
    os.replace(lib + ".tmp", lib)
    return lib


def test_abi_validation_under_asan_ubsan():
    rt = _clang_runtime()
    lib = _sanitized_libfuse()
    code = ("import sys, pytest\n"
            "from memory_bound_amd import api\n"
            f"api.LIB_PATH = {lib!r}\n"
            "sys.exit(pytest.main(['-x', '-q', '-p', 'no:cacheprovider', '-m', 'not gpu', 'tests/test_abi.py']))\n")
    r = _run_python(code, {"LD_PRELOAD": rt, "LD_LIBRARY_PATH": os.path.dirname(rt) + ":" +
                           os.environ.get("LD_LIBRARY_PATH", "")})
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout
