"""CPU AddressSanitizer + UndefinedBehaviorSanitizer runs.

- The oracle (oracle/tb_oracle.c) built with gcc's -fsanitize=address,undefined
  runs its pinned tests (tests/test_oracle_*.py) in a child process with the
  sanitizer runtime preloaded; any report aborts the child.
- libtb's host code built with the same sanitizers (device code unchanged)
  runs tests/test_abi.py: symbol export, status strings, workspace queries at
  ordinary and extreme sizes and the argument validation that rejects bad
  calls before anything is enqueued (no GPU is used).
- First, a planted heap overflow and a planted signed overflow in a scratch C
  file built with the same flags must be reported, so a silent run means the
  sanitizers were live."""
import glob
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")


def _gcc_asan():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                       text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _clang_asan():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    found = sorted(glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    return found[-1] if found else None


def _child(code, preload, extra_env=None, timeout=600):
    # the child's pytest runs with -s: a sanitizer report ends the process at
    # once, before pytest would print output it had captured
    env = dict(os.environ)
    env.update({"LD_PRELOAD": preload,
                "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
                "PYTHONDONTWRITEBYTECODE": "1"})
    env.update(extra_env or {})
    r = subprocess.run([sys.executable, "-c", textwrap.dedent(code)], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


def _reports(out):
    return [l for l in out.splitlines()
            if "runtime error:" in l or "ERROR: AddressSanitizer" in l]


@pytest.fixture(scope="module")
def gcc_asan():
    p = _gcc_asan()
    if p is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return p


def test_planted_errors_are_reported(gcc_asan, tmp_path):
    src = tmp_path / "planted.c"
    src.write_text(textwrap.dedent("""\
        #include <stdlib.h>
        int heap_read(int i) { int *p = malloc(4 * sizeof(int)); p[0] = 1;
                               int v = p[i]; free(p); return v; }
        int add(int a, int b) { return a + b; }
        """))
    so = str(tmp_path / "libplanted.so")
    subprocess.check_call(["gcc", "-shared", "-fPIC"] + _oracle_flags() + ["-o", so, str(src)])
    code = """
        import ctypes, sys
        L = ctypes.CDLL(%r)
        print("in bounds", L.heap_read(%d), flush=True)
        L.%s
    """
    rc, out = _child(code % (so, 0, "heap_read(4)"), gcc_asan)
    # reported by ASan (heap-buffer-overflow) or first by UBSan's object-size check
    assert rc != 0 and _reports(out) and ("heap-buffer-overflow" in out or "load of" in out), \
        out[-2000:]
    rc, out = _child(code % (so, 0, "add(2147483647, 1)"), gcc_asan)
    assert rc != 0 and "signed integer overflow" in out, out[-2000:]


def _oracle_flags():
    sys.path.insert(0, ROOT)
    from oracle import oracle as o
    return list(o.SANITIZE_FLAGS)


def test_oracle_pins_under_sanitizers(gcc_asan, tmp_path):
    sys.path.insert(0, ROOT)
    from oracle import oracle as o
    so = str(tmp_path / "libtb_oracle_san.so")
    o.build(path=so, extra_flags=o.SANITIZE_FLAGS)
    files = sorted(glob.glob(os.path.join(TESTS, "test_oracle_*.py")))
    code = """
        import sys
        import pytest
        sys.exit(pytest.main(["-q", "-x", "-s", "-p", "no:cacheprovider", "-m", "not gpu"] + %r))
    """ % files
    rc, out = _child(code, gcc_asan, {"TB_ORACLE_LIB": so}, timeout=900)
    assert not _reports(out), "\n".join(_reports(out)[:20])
    assert rc == 0, out[-3000:]
    assert " passed" in out


def test_abi_validation_under_sanitizers(tmp_path):
    rt = _clang_asan()
    if rt is None:
        pytest.skip("ROCm clang's AddressSanitizer runtime is not installed")
    sys.path.insert(0, ROOT)
    from learned_kv_cache_amd import build as b
    so = str(tmp_path / "libtb_san.so")
    b.build(lib=so, objdir=str(tmp_path / "obj"), extra_flags=b.HOST_SANITIZE_FLAGS)
    code = """
        import sys
        import pytest
        import learned_kv_cache_amd as tb
        tb.LIB_PATH = %r
        sys.exit(pytest.main(["-q", "-x", "-s", "-p", "no:cacheprovider", %r]))
    """ % (so, os.path.join(TESTS, "test_abi.py"))
    rc, out = _child(code, rt)
    assert not _reports(out), "\n".join(_reports(out)[:20])
    assert rc == 0, out[-3000:]
    assert " passed" in out
