"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host code only, gcc):
oracle.c is built with -fsanitize=address,undefined (every finding fatal) and the whole pin
suite runs against that build in a child process, with the ASan runtime preloaded into the
interpreter. Any out-of-bounds access, use after free or undefined operation in the oracle
fails this test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(shutil.which("gcc") is None or _runtime("libasan.so") is None,
                    reason="gcc with the ASan runtime is needed")
def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_asan.so")
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-fPIC", "-shared",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                           "-o", lib, SRC, "-lm"])
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": _runtime("libasan.so"),
        # the interpreter and torch are not instrumented: no leak report at exit, and their
        # own allocator pairs are not the subject here
        "ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0:new_delete_type_mismatch=0:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "CSA_ORACLE_LIB": lib,
        "OMP_NUM_THREADS": "4",
    })
    probe = ("import ctypes, oracle; oracle.lib(); "
             "assert oracle.LIB_PATH == %r; assert hasattr(ctypes.CDLL(None), '__asan_init')" % lib)
    subprocess.check_call([sys.executable, "-c", probe], cwd=ROOT, env=env)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
