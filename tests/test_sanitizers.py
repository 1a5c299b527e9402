"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The oracle (plain C) is rebuilt with gcc -fsanitize=address,undefined and its pin and
  planted-mistake tests run against it in a child process (the ASan runtime preloaded).
- libsdpa's host side (argument validation, workspace sizing, status strings: everything
  that runs before a launch) is rebuilt with -fsanitize=address,undefined applied to the
  host pass only (-Xarch_host; the gfx950 code is unchanged) and the C-ABI tests run
  against it in a child process.
Any sanitizer report aborts the child (UBSan without recovery), which fails the test.
"""
import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def run_child(code: str, preload: str, env_extra=None, timeout=900):
    env = dict(os.environ)
    env["LD_PRELOAD"] = preload
    # Python itself keeps its allocations until exit: leak reports are not ours
    env["ASAN_OPTIONS"] = "detect_leaks=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    env.update(env_extra or {})
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=timeout)
    out = r.stdout + r.stderr
    assert not any(x in out for x in REPORTS), out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's ASan runtime not available")
    lib = str(tmp_path / "liboracle_asan.so")
    subprocess.check_call([gcc, "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", "-shared", "-fPIC", "-o", lib,
                           os.path.join(ROOT, "oracle", "sdpa_oracle.c"), "-lpthread", "-lm"])
    code = f"""
import os, sys
sys.path.insert(0, {ROOT!r})
import oracle
oracle._LIB_PATH = {lib!r}
os.utime(oracle._LIB_PATH)  # newer than the source: used as built
import pytest
rc = pytest.main(['-q', '-x', '-m', 'not gpu', '-p', 'no:cacheprovider',
                  'tests/test_oracle_pins.py', 'tests/test_oracle_mutations.py'])
assert oracle._lib is not None and oracle._lib._name == {lib!r}
sys.exit(rc)
"""
    out = run_child(code, asan)
    assert " passed" in out


def _clang_asan_runtime():
    for pat in ("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so",
                "/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"):
        hits = sorted(glob.glob(pat))
        if hits:
            return hits[-1]
    return None


def test_c_abi_host_code_under_asan_ubsan(tmp_path):
    from scaled_dot_product_19_amd import build as B
    try:
        cc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("clang's ASan runtime not available")
    # sanitizers on the host pass only: each flag right after -Xarch_host
    san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
              "-fno-omit-frame-pointer", "-shared-libsan"):
        san += ["-Xarch_host", f]

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        subprocess.check_call([cc] + B.common_flags() + B.EXTRA_FLAGS.get(src, []) + san +
                              ["-c", os.path.join(B.CSRC, src), "-o", obj],
                              stderr=subprocess.DEVNULL)
        return obj

    with concurrent.futures.ThreadPoolExecutor(min(8, len(B.SOURCES))) as ex:
        objs = list(ex.map(compile_one, B.SOURCES))
    lib = str(tmp_path / "libsdpa_asan.so")
    subprocess.check_call([cc, "--offload-arch=" + B.ARCH, "-shared", "-fPIC"] + san +
                          ["-o", lib] + objs, stderr=subprocess.DEVNULL)
    code = f"""
import sys
sys.path.insert(0, {ROOT!r})
from scaled_dot_product_19_amd import sdpa
sdpa._LIB_PATH = {lib!r}
sdpa.load()
import pytest
sys.exit(pytest.main(['-q', '-x', '-m', 'not gpu', '-p', 'no:cacheprovider',
                      'tests/test_abi.py']))
"""
    ld = os.path.dirname(rt) + (":" + os.environ["LD_LIBRARY_PATH"]
                                 if os.environ.get("LD_LIBRARY_PATH") else "")
    out = run_child(code, rt, {"LD_LIBRARY_PATH": ld})
    assert " passed" in out
