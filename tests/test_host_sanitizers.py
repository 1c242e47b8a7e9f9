"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Two builds, each into this test's temporary directory (never into the tree):
  * oracle.c with gcc -fsanitize=address,undefined; the oracle's pins (tests/test_oracle_pins.py) then run against it
    in a fresh interpreter with gcc's libasan preloaded;
  * libbcjr.so with its C-ABI translation unit (every argument check, workspace plan and dispatch decision of the
    library's host side) compiled with hipcc -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined and linked
    with the kernels' objects of the last build; the host tests of the C-ABI (tests/test_abi_host.py) then run against
    it with clang's ASan runtime preloaded.
UBSan findings abort (-fno-sanitize-recover); ASan's leak check is off (the interpreter itself holds memory at exit).
A control for each setup plants a one-past-the-end heap read in a throwaway snippet built the same way and checks
that the run aborts with ASan's report, so a pass means the sanitizers were live.

The same sessions by hand, from the repository root:
    python -m differentiable_bcjr_amd.build
    python -m pytest -q tests/test_host_sanitizers.py
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "OMP_NUM_THREADS": "4"}

PLANTED = r"""
#include <stdlib.h>
#ifdef __cplusplus
extern "C"
#endif
int planted_overflow(int n) {
    volatile int* a = (volatile int*)malloc(n * sizeof(int));
    for (int i = 0; i < n; ++i) a[i] = i;
    int s = a[n];   /* one past the end */
    free((void*)a);
    return s;
}
"""


def _gcc_asan():
    return subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()


def _run(env_extra, args, timeout=900):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


def _call_planted(lib, preload):
    code = f"import ctypes; ctypes.CDLL({lib!r}).planted_overflow(8)"
    return _run({"LD_PRELOAD": preload}, ["-c", code], timeout=120)


def _pytest(env_extra, test_file):
    return _run(env_extra, ["-m", "pytest", "-q", "-p", "no:cacheprovider", os.path.join("tests", test_file)])


@pytest.mark.slow
def test_oracle_pins_under_gcc_sanitizers(tmp_path):
    import oracle

    src = tmp_path / "planted.c"
    src.write_text(PLANTED)
    ctl = str(tmp_path / "libplanted.so")
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", *oracle.SANITIZE_FLAGS, "-o", ctl, str(src)])
    r = _call_planted(ctl, _gcc_asan())
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]

    lib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    r = _pytest({"LD_PRELOAD": _gcc_asan(), "ORACLE_LIB": lib}, "test_oracle_pins.py")
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


@pytest.mark.slow
def test_abi_host_side_under_clang_sanitizers(tmp_path):
    from differentiable_bcjr_amd import build as B

    rt = B.asan_runtime()
    src = tmp_path / "planted.cpp"
    src.write_text(PLANTED)
    ctl = str(tmp_path / "libplanted.so")
    subprocess.check_call([B.hipcc(), "-O2", "-fPIC", "-shared", *B.SANITIZE_HOST_FLAGS, "-o", ctl, str(src)])
    r = _call_planted(ctl, rt)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]

    if not all(os.path.exists(os.path.join(B.BUILD_DIR, s + ".o")) for s in B.SOURCES if s != "bcjr_abi.cpp"):
        B.build()
    lib = B.build_sanitized(str(tmp_path / "libbcjr_san.so"))
    r = _pytest({"LD_PRELOAD": rt, "BCJR_LIB": lib}, "test_abi_host.py")
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
