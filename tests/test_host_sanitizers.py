"""CPU: the host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Three host parts take untrusted sizes and indices: the split-KV planner and
the argument checks of the C ABI (``csrc/planner.cpp``, ``csrc/api.cpp``,
``csrc/noalloc.hip``, inside ``libmla_decode.so``), and the fp64 oracle
(``oracle/mla_oracle.c``).  Each is rebuilt with ASan + UBSan on its host code
(device code is not instrumented; nothing here needs a GPU) and the existing
CPU tests of that part run against the instrumented build in a child process
that preloads the matching sanitizer runtime (clang's for the hipcc build,
gcc's for the oracle), with every report fatal.  A planted heap overflow and a
planted signed overflow check that the harness does catch errors.
"""
import glob
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_paged_kv_decode_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "OMP_NUM_THREADS": "4"}


def _clang_asan_runtime():
    c = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return c[-1] if c else None


def _gcc_runtimes():
    out = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                           text=True).stdout.strip()
        if not os.path.isabs(p) or not os.path.exists(p):
            return None
        out.append(p)
    return out


def _child(preload, code):
    env = dict(os.environ, LD_PRELOAD=" ".join(preload), **SAN_ENV)
    return subprocess.run([sys.executable, "-c", textwrap.dedent(code)], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=1500)


def _clean(r):
    text = r.stdout + r.stderr
    assert "runtime error" not in text and "AddressSanitizer" not in text, text[-4000:]
    assert r.returncode == 0, text[-4000:]
    return text


# host instrumentation only: each -fsanitize flag applies to the host pass
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def sanitized_library(tmp_path_factory):
    if not os.path.exists(HIPCC) or _clang_asan_runtime() is None:
        pytest.skip("hipcc or the clang ASan runtime missing")
    out = str(tmp_path_factory.mktemp("san") / "libmla_decode_san.so")
    srcs = [os.path.join(CSRC, s) for s in ("api.cpp", "planner.cpp", "kernels.hip",
                                            "append.hip", "peaks.hip", "noalloc.hip")]
    cmd = ([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument", "-Wno-inline-asm",
            "-I", os.path.join(ROOT, "include")] + SAN_HOST + srcs + ["-o", out])
    subprocess.run(cmd, check=True, capture_output=True)
    return out


def test_planner_and_abi_clean_under_asan_ubsan(sanitized_library):
    r = _child([_clang_asan_runtime()], """
        import sys
        import mla_paged_kv_decode_amd as m
        m.load_library(%r)
        import pytest
        sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu",
                              "tests/test_abi_planner.py", "tests/test_zz_no_alloc.py"]))
        """ % sanitized_library)
    text = _clean(r)
    assert " passed" in text and " failed" not in text


def test_oracle_clean_under_asan_ubsan(tmp_path):
    rts = _gcc_runtimes()
    if rts is None:
        pytest.skip("gcc sanitizer runtimes missing")
    so = str(tmp_path / "libmla_oracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-pthread",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-fno-fast-math", "-ffp-contract=off",
                    os.path.join(ROOT, "oracle", "mla_oracle.c"), "-o", so, "-lm"],
                   check=True, capture_output=True)
    r = _child(rts, """
        import sys
        import oracle
        oracle._LIB = %r       # loaded as it is: newer than the source, never rebuilt
        import pytest
        rc = pytest.main(["-q", "-p", "no:cacheprovider", "tests/test_oracle_pins.py"])
        assert oracle._LIB == %r
        sys.exit(rc)
        """ % (so, so))
    text = _clean(r)
    assert " passed" in text and " failed" not in text


PLANTED = r"""
#include <stdint.h>
#include <stdlib.h>
int heap_overflow(int n) { int* p = (int*)malloc(4 * n); int v = p[n]; free(p); return v; }
int32_t add_overflow(int32_t a) { return a + INT32_MAX; }
"""


@pytest.mark.parametrize("call,report", [("heap_overflow(4)", "heap-buffer-overflow"),
                                         ("add_overflow(7)", "runtime error")])
def test_harness_reports_planted_errors(tmp_path, call, report):
    rts = _gcc_runtimes()
    if rts is None:
        pytest.skip("gcc sanitizer runtimes missing")
    src = tmp_path / "planted.c"
    src.write_text(PLANTED)
    so = str(tmp_path / "libplanted.so")
    subprocess.run(["gcc", "-O0", "-g", "-fPIC", "-shared", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", str(src), "-o", so], check=True,
                   capture_output=True)
    r = _child(rts, """
        import ctypes
        lib = ctypes.CDLL(%r)
        lib.%s
        """ % (so, call))
    assert r.returncode != 0 and report in (r.stdout + r.stderr)
