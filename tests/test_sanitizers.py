"""Address and undefined-behaviour sanitizer runs of the host code, on the CPU (no GPU involved).

1. The fp64 oracle built with gcc -fsanitize=address,undefined and driven through its pin tests
   (tests/test_oracle_*pins.py: decode, rotary decode, prefill, encode, append, flat attention and
   the fit on small, ragged and empty inputs).
2. liblla.so with the sanitizers on its host pass only (argument validation, split planning, the
   ABI's host helpers; the gfx950 device code is compiled as usual), driven through the ABI's
   validation tests (tests/test_abi.py), which never launch a kernel.

Each runs in a subprocess with the matching sanitizer runtime preloaded (the interpreter itself is
not instrumented); any sanitizer report, or a failing test, fails here.  The instrumented builds
go to _build/sanitize/ and are rebuilt when a source changes.
"""
import glob
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
CSRC = os.path.join(ROOT, "looped_transformer_kv_amd", "csrc")
ORACLE_SRC = os.path.join(ROOT, "oracle", "lla_oracle.c")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG_ASAN = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")

PLUGIN = '''
import os
def pytest_configure(config):
    if os.environ.get("SAN_ORACLE_LIB"):
        from oracle import build
        build.LIB = os.environ["SAN_ORACLE_LIB"]
    if os.environ.get("SAN_LLA_LIB"):
        from looped_transformer_kv_amd import lla
        lla.LIB_PATH = os.environ["SAN_LLA_LIB"]
'''


def _digest(paths, extra=""):
    h = hashlib.sha256(extra.encode())
    for p in sorted(paths):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _gcc_runtime(name):
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()


def _run_pytest(tests, env_extra):
    os.makedirs(OUT, exist_ok=True)
    with open(os.path.join(OUT, "san_plugin.py"), "w") as f:
        f.write(PLUGIN)
    env = dict(os.environ)
    env.update(env_extra)
    env["PYTHONPATH"] = os.pathsep.join([OUT, ROOT, os.path.join(ROOT, "tests")] +
                                        [env.get("PYTHONPATH", "")])
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "2"
    env["HIP_VISIBLE_DEVICES"] = ""             # host code only: never reach a device
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "san_plugin",
                        "-p", "no:cacheprovider", "-m", "not gpu"] + tests,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    return out


def test_oracle_under_asan_ubsan():
    lib = os.path.join(OUT, f"liblla_oracle_san_{_digest([ORACLE_SRC])}.so")
    if not os.path.exists(lib):
        os.makedirs(OUT, exist_ok=True)
        subprocess.run(["gcc", "-O1", "-g", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                        "-std=c99", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined", "-o", lib + ".tmp", ORACLE_SRC, "-lm"],
                       check=True)
        os.replace(lib + ".tmp", lib)
    preload = ":".join([_gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")])
    tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*pins.py")))
    _run_pytest(tests, {"LD_PRELOAD": preload, "SAN_ORACLE_LIB": lib})


@pytest.mark.skipif(not CLANG_ASAN, reason="clang's address-sanitizer runtime is not installed")
def test_host_validation_under_asan_ubsan():
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    headers = sorted(glob.glob(os.path.join(CSRC, "*.h"))) + [os.path.join(ROOT, "include",
                                                                           "lla.h")]
    lib = os.path.join(OUT, f"liblla_san_{_digest(srcs + headers)}.so")
    if not os.path.exists(lib):
        os.makedirs(OUT, exist_ok=True)
        flags = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
                 "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                 "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all",
                 "-Xarch_host", "-fno-omit-frame-pointer",
                 "-I", os.path.join(ROOT, "include")]
        procs, objs = [], []
        for s in srcs:
            o = os.path.join(OUT, os.path.basename(s)[:-4] + ".san.o")
            objs.append(o)
            procs.append(subprocess.Popen([HIPCC] + flags + ["-c", s, "-o", o],
                                          stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
        for p in procs:
            out = p.communicate()[0]
            assert p.returncode == 0, out.decode()[-4000:]
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                        "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                        "-fsanitize=undefined", "-shared-libsan", "-o", lib + ".tmp"] + objs,
                       check=True, capture_output=True)
        os.replace(lib + ".tmp", lib)
        for o in objs:
            os.remove(o)
    _run_pytest([os.path.join(ROOT, "tests", "test_abi.py")],
                {"LD_PRELOAD": CLANG_ASAN[0], "SAN_LLA_LIB": lib})
