"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only; no GPU code runs).

- The oracle's C sources (oracle/fa_ref*.c) are built with gcc -fsanitize=address,undefined into a
  library of their own, and the oracle's pin tests run against that build in a child Python process
  (the ASan runtime preloaded, FA_ORACLE_LIB naming the build). A planted out-of-bounds call, an
  output buffer one row too short, must be caught, which shows the sanitizer is live.
- libfa's host code (argument checks, plans, status strings of every entry point) is built with the
  sanitizers on the host pass only (each -fsanitize= behind -Xarch_host; the gfx950 device code is
  built as usual and never runs here), linked into the plain C program tests/c_consumer.c (built with
  clang and the same sanitizers), and that program's host checks run with leak detection on.
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ORACLE_SRC = [os.path.join(ROOT, "oracle", n) for n in ("fa_ref.c", "fa_ref_bwd.c", "fa_ref_sparse.c")]
PIN_TESTS = ["test_oracle_pins.py", "test_oracle_bwd_pins.py", "test_oracle_sparse_pins.py",
             "test_oracle_splitkv_pins.py", "test_oracle_fp8_pins.py", "test_oracle_properties.py"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r


@pytest.fixture(scope="module")
def oracle_asan(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("asan") / "liboracle_asan.so")
    r = run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
             "-Wall", "-Wextra", "-o", out, *ORACLE_SRC, "-lm"])
    assert r.returncode == 0, r.stderr
    libasan = run(["gcc", "-print-file-name=libasan.so"]).stdout.strip()
    assert os.path.isabs(libasan) and os.path.exists(libasan), libasan
    env = dict(os.environ, FA_ORACLE_LIB=out, LD_PRELOAD=libasan, **SAN_ENV)
    return out, env


def test_oracle_pins_under_asan_ubsan(oracle_asan):
    lib, env = oracle_asan
    r = run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
             *[os.path.join(HERE, t) for t in PIN_TESTS]], env=env, cwd=ROOT, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout and "failed" not in r.stdout
    # the child really loaded the sanitized build
    r = run([sys.executable, "-c", "import oracle; oracle._load(); print(oracle._LIB_PATH)"], env=env,
            cwd=ROOT, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == lib, r.stderr


def test_asan_catches_a_planted_overflow(oracle_asan):
    # fa_ref_fwd writing O of 2 rows into a buffer sized for 1: a heap-buffer-overflow under ASan
    _, env = oracle_asan
    # (the buffers come from malloc, which ASan tracks; Python's small-object allocator it does not)
    code = (
        "import ctypes, numpy as np, oracle\n"
        "L = oracle._load()\n"
        "libc = ctypes.CDLL(None); libc.malloc.restype = ctypes.c_void_p\n"
        "libc.malloc.argtypes = [ctypes.c_size_t]\n"
        "dp = ctypes.POINTER(ctypes.c_double)\n"
        "o = ctypes.cast(libc.malloc(8 * 64), dp); lse = ctypes.cast(libc.malloc(8 * 2), dp)\n"
        "q = np.zeros((1, 1, 2, 64), np.uint16)\n"
        "p = q.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))\n"
        "L.fa_ref_fwd(p, p, p, o, lse, 1, 1, 2, 64, 1, 0.125, 1)\n"
        "print('not caught')\n")
    r = run([sys.executable, "-c", code], env=env, cwd=ROOT, timeout=120)
    assert r.returncode != 0 and "not caught" not in r.stdout
    assert "AddressSanitizer" in r.stderr and "buffer-overflow" in r.stderr, r.stderr[-2000:]


@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "bin", "hipcc")), reason="hipcc not found")
def test_libfa_host_checks_under_asan_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from exact_tiled_attention_07_amd import build as fa_build

    lib = str(tmp_path / "libfa.so")
    flags = ["-O1", "-g", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all"]
    fa_build.build(extra_flags=flags, out=lib)
    exe = str(tmp_path / "c_consumer")
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    r = run([clang, "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
             "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(ROCM, "include"),
             os.path.join(HERE, "c_consumer.c"), "-o", exe, "-L", str(tmp_path), "-lfa",
             "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{tmp_path}",
             f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"])
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS=SAN_ENV["UBSAN_OPTIONS"])
    r = run([exe, "host"], env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")
