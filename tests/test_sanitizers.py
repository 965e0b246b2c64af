"""Host sanitizers, CPU only: AddressSanitizer and UndefinedBehaviorSanitizer builds of the C
oracle and of the C ABI's host code, with the oracle pins and the ABI tests run against them.

The oracle (oracle/gdr_oracle.c) is compiled with clang -fsanitize=address,undefined; the
library's host side (validation and dispatch, gdr_api.hip) is compiled with the same
sanitizers on its host pass only and linked with the regular objects of the other sources (no
GPU code runs on the CPU: every ABI test call is rejected or is a no-op before any launch).
The tests then run in a child process with the sanitizer runtime preloaded, and any report
fails the run (UBSan halts on its first error)."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = "/opt/rocm/llvm"
CLANG = os.path.join(LLVM, "bin", "clang")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _runtime():
    found = sorted(glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    return found[-1] if found else None


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    rt = _runtime()
    objs = sorted(glob.glob(os.path.join(ROOT, "_build", "*.hip.o")))
    if not (os.path.exists(CLANG) and os.path.exists(HIPCC) and rt):
        pytest.skip("clang / hipcc / the ASan runtime are not available")
    objs = [o for o in objs if not o.endswith("gdr_api.hip.o")]
    if not objs:
        pytest.skip("the regular library build (_build/*.hip.o) is not there")
    d = tmp_path_factory.mktemp("sanitizers")
    oracle_so = str(d / "libgdr_oracle_san.so")
    subprocess.run([CLANG, "-O1", "-g", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    f"-Wl,-rpath,{LLVM}/lib", "-o", oracle_so, os.path.join(ROOT, "oracle", "gdr_oracle.c"), "-lm"],
                   check=True, capture_output=True)
    sys.path.insert(0, os.path.join(ROOT, "gated_delta_rule_15_amd"))
    import build as libbuild  # the library's own build flags
    api_o = str(d / "gdr_api_san.o")
    subprocess.run([HIPCC, *libbuild.FLAGS, "-g",
                    "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
                    "-Xarch_host", "-fno-omit-frame-pointer",
                    "-c", os.path.join(ROOT, "gated_delta_rule_15_amd", "csrc", "gdr_api.hip"), "-o", api_o],
                   check=True, capture_output=True)
    lib_so = str(d / "libgdr_san.so")
    subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={libbuild.ARCH}", "-o", lib_so, api_o, *objs],
                   check=True, capture_output=True)
    env = dict(os.environ, LD_PRELOAD=rt, GDR_ORACLE_LIBRARY=oracle_so, GDR_LIBRARY=lib_so,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=24", OMP_NUM_THREADS="4")
    return env


def _run(env, *tests):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *[os.path.join(ROOT, "tests", t) for t in tests]],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_under_sanitizers(sanitized):
    out = _run(sanitized, "test_oracle_pins.py", "test_oracle_gdp.py", "test_oracle_gdn2.py")
    print(out.strip().splitlines()[-1])


def test_abi_under_sanitizers(sanitized):
    out = _run(sanitized, "test_abi.py")
    print(out.strip().splitlines()[-1])


PLANTED = """
import ctypes, numpy as np, oracle
lib = oracle._load()
P = ctypes.c_void_p
# the shapes say 8 tokens; the token arrays hold 4, so the oracle reads past their end
T, dk, dv = 8, 64, 64
q = np.zeros((4, dk), np.float32); k = q.copy(); v = q.copy(); g = np.zeros(4, np.float32); b = g.copy()
o = np.zeros((T, dv), np.float64); S = np.zeros((dv, dk), np.float64)
lib.oracle_gdr_forward(1, T, dk, dv, 0, *(a.ctypes.data_as(P) for a in (q, k, v, g, b)), None,
                       o.ctypes.data_as(P), S.ctypes.data_as(P), 1)
"""


def test_sanitizers_catch_a_planted_overflow(sanitized):
    """Control: the same sanitized oracle, called with arrays shorter than the shapes it is
    given, must stop with a heap-buffer-overflow report (else the two tests above prove
    nothing)."""
    r = subprocess.run([sys.executable, "-c", PLANTED], cwd=ROOT, env=dict(sanitized, PYTHONPATH=ROOT),
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0, r.stderr[-2000:]
    assert "heap-buffer-overflow" in r.stderr and "oracle_gdr_forward" in r.stderr, r.stderr[-2000:]
