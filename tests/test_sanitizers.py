"""Host-side sanitizer builds (CPU only, no GPU):

* the CPU oracle (oracle/gqref.c) under AddressSanitizer + LeakSanitizer +
  UBSan, driven through every entry point by tests/sanitize_oracle_driver.c
  (leaks checked), and as a shared library under ASan + UBSan running the
  oracle's pins (tests/test_oracle_*.py) in a child process;
* the C ABI's host code (csrc/api.hip: argument validation, size queries,
  dispatch) built with ASan + UBSan for the host side only, running the
  ABI tests (tests/test_abi.py, which reach no kernel launch) in a child
  process.

A planted heap overflow in a separate probe checks that the toolchain's
sanitizer is really active.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer", "-g", "-O1"]
ORACLE_FLAGS = ["-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")
HIPCC = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")


def _run(cmd, env=None, timeout=600):
    return subprocess.run(cmd, capture_output=True, text=True, env=env,
                          timeout=timeout, cwd=ROOT)


def _gcc_runtime(name):
    return _run(["gcc", f"-print-file-name={name}"]).stdout.strip()


def _child_env(**extra):
    env = dict(os.environ)
    env.pop("LD_PRELOAD", None)
    env.update(extra)
    return env


@pytest.fixture(scope="module")
def outdir():
    os.makedirs(OUT, exist_ok=True)
    return OUT


def test_planted_overflow_is_caught(outdir):
    src = os.path.join(outdir, "planted.c")
    with open(src, "w") as f:
        f.write("#include <stdlib.h>\nint main(void) {\n"
                "  volatile int *a = malloc(4 * sizeof(int));\n"
                "  int i = 4;\n  a[i] = 1;\n  free((void *)a);\n  return 0;\n}\n")
    exe = os.path.join(outdir, "planted")
    r = _run(["gcc", *SAN, src, "-o", exe])
    assert r.returncode == 0, r.stderr
    r = _run([exe])
    assert r.returncode != 0
    # UBSan's object-size check or ASan's shadow check, whichever fires first
    assert "heap-buffer-overflow" in r.stderr or "insufficient space" in r.stderr


def test_oracle_driver_asan_lsan_ubsan(outdir):
    exe = os.path.join(outdir, "oracle_driver")
    r = _run(["gcc", *SAN, *ORACLE_FLAGS,
              os.path.join(ROOT, "tests", "sanitize_oracle_driver.c"),
              os.path.join(ROOT, "oracle", "gqref.c"), "-o", exe, "-lm"])
    assert r.returncode == 0, r.stderr
    r = _run([exe], env=_child_env(ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                                   OMP_NUM_THREADS="4"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "every entry point ran" in r.stdout


def test_oracle_pins_under_asan_ubsan(outdir):
    lib = os.path.join(outdir, "libgqref_asan.so")
    r = _run(["gcc", *SAN, *ORACLE_FLAGS, "-fPIC", "-shared",
              os.path.join(ROOT, "oracle", "gqref.c"), "-o", lib, "-lm"])
    assert r.returncode == 0, r.stderr
    pins = sorted(os.path.join("tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                  if f.startswith("test_oracle_") and f.endswith(".py"))
    env = _child_env(LD_PRELOAD=f"{_gcc_runtime('libasan.so')} {_gcc_runtime('libubsan.so')}",
                     ASAN_OPTIONS="detect_leaks=0", GQREF_LIBRARY=lib,
                     OMP_NUM_THREADS="4")
    r = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
              "-m", "not gpu", *pins], env=env, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout


def test_c_abi_host_code_under_asan_ubsan(outdir):
    from communication_efficient_gradient_amd import build as lib_build
    objdir = os.path.join(ROOT, "_build", "libgq")
    others = [s[:-4] for s in lib_build.SOURCES if s != "api.hip"]
    if not all(os.path.exists(os.path.join(objdir, o + ".o")) for o in others):
        lib_build.build()
    api_o = os.path.join(outdir, "api_asan.o")
    host_san = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined",
                 "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"):
        host_san += ["-Xarch_host", flag]
    flags = [f for f in lib_build.HIPFLAGS if f not in ("-O3",)]
    r = _run([HIPCC, *flags, "-O1", "-g", *host_san, "-c",
              os.path.join(ROOT, "communication_efficient_gradient_amd", "csrc", "api.hip"),
              "-o", api_o])
    assert r.returncode == 0, r.stderr
    lib = os.path.join(outdir, "libgq_asan.so")
    r = _run([CLANG, "-shared", "-fPIC", "-fsanitize=address,undefined",
              "-shared-libsan", api_o,
              *[os.path.join(objdir, o + ".o") for o in others],
              f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", lib])
    assert r.returncode == 0, r.stderr
    rt = _run([os.path.join(ROCM, "llvm", "bin", "clang"),
               "-print-file-name=libclang_rt.asan-x86_64.so"]).stdout.strip()
    assert os.path.exists(rt), rt
    env = _child_env(LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0", GQ_LIBRARY=lib)
    r = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
              "-m", "not gpu", os.path.join("tests", "test_abi.py")], env=env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout
