"""The oracle and the C ABI's host-side validation under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU).

* oracle/ss_oracle.c is rebuilt with -fsanitize=address,undefined and every oracle pin
  runs against that build (threaded paths included);
* selective_state_space_85_amd/csrc/ss_api.cpp (argument validation, plans, workspace
  layouts) is rebuilt the same way with stub kernel launchers
  (tests/sanitize/launch_stubs.cpp) and tests/test_abi.py runs against it;
* a planted out-of-bounds write shows the sanitizer is live.
Each run is a subprocess with the sanitizer runtime preloaded; any report fails it.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="gcc/g++ not available")


def _asan_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("no libasan runtime")
    return path


def _run(args, env_extra, timeout=600):
    env = dict(os.environ)
    env.update({"LD_PRELOAD": _asan_runtime(), "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    env.update(env_extra)
    return subprocess.run(args, capture_output=True, text=True, env=env, timeout=timeout, cwd=ROOT)


def test_sanitizer_is_live(tmp_path):
    """A planted heap overflow in a sanitized library is reported (by AddressSanitizer, or
    first by UndefinedBehaviorSanitizer's object-size check) and aborts the run."""
    src = tmp_path / "bad.c"
    src.write_text("#include <stdlib.h>\nint bad(int i) { int* p = malloc(4 * sizeof(int));"
                   " p[i] = 1; int v = p[0]; free(p); return v; }\n")
    lib = tmp_path / "libbad.so"
    subprocess.run(["gcc", "-shared", "-fPIC"] + SAN + ["-o", str(lib), str(src)], check=True)
    code = "import ctypes, sys; l = ctypes.CDLL(sys.argv[1]); l.bad(4)"
    r = _run([sys.executable, "-c", code, str(lib)], {})
    assert r.returncode != 0, r.stderr[-2000:]
    assert "heap-buffer-overflow" in r.stderr or "insufficient space" in r.stderr, r.stderr[-2000:]


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc"] + SAN + ["-ffp-contract=off", "-std=c11", "-fPIC", "-shared", "-o", str(lib),
                                    os.path.join(ROOT, "oracle", "ss_oracle.c"), "-lm", "-lpthread"], check=True)
    code = ("import sys; sys.path[:0] = [%r, %r]\n"
            "import oracle, pins\n"
            "orc = oracle.OracleLib(sys.argv[1])\n"
            "for pin in pins.ALL_PINS:\n"
            "    pin(orc)\n"
            "print('pins:', len(pins.ALL_PINS))\n") % (ROOT, TESTS)
    r = _run([sys.executable, "-c", code, str(lib)], {})
    assert r.returncode == 0 and "pins:" in r.stdout, (r.stdout[-1000:], r.stderr[-3000:])


def _host_lib(tmp_path):
    lib = tmp_path / "libssscan_host_san.so"
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-shared"] + SAN +
                   ["-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "selective_state_space_85_amd", "csrc"),
                    os.path.join(ROOT, "selective_state_space_85_amd", "csrc", "ss_api.cpp"),
                    os.path.join(TESTS, "sanitize", "launch_stubs.cpp"), "-o", str(lib)], check=True)
    return lib


def test_abi_validation_under_sanitizers(tmp_path):
    lib = _host_lib(tmp_path)
    r = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "sanitize.abi_plugin", "-p", "no:cacheprovider",
              os.path.join(TESTS, "test_abi.py"), os.path.join(TESTS, "test_zz_no_alloc.py"), "-m", "not gpu"],
             {"SS_SANITIZED_LIB": str(lib), "PYTHONPATH": TESTS + os.pathsep + ROOT})
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout


def test_hip_failure_path(tmp_path):
    """Valid calls whose launches fail (the stub launchers return the code in
    SS_STUB_LAUNCH_ERROR) return SS_ERR_HIP and leave the HIP code in ss_last_hip_error:
    the scan with and without chunks, the allocation-free scan, the step, the backward,
    the conv1d and the multi-head recurrence."""
    lib = _host_lib(tmp_path)
    code = ("import ctypes, sys; sys.path[:0] = [%r, %r]\n"
            "import sanitize.abi_plugin\n"
            "from selective_state_space_85_amd import _lib\n"
            "import test_abi as t\n"
            "lib = _lib.load()\n"
            "assert lib.ss_last_hip_error() == 0\n"
            "assert t.call_scan(lib) == 4, 'one chunk'\n"
            "assert lib.ss_last_hip_error() == 17\n"
            "assert t.call_scan(lib, chunk=64) == 4, 'chunked'\n"
            "assert t.call_scan(lib, chunk=1024, seqlen=4096) == 4, 'emit first'\n"
            "a = t.addr\n"
            "assert lib.ss_scan_fwd_noalloc(a(0), a(1), a(2), a(3), a(4), None, None, None, a(5), None,"
            " 2, 512, 64, 16, t.BF16, None) == 4, 'allocation-free'\n"
            "assert t.call_step(lib) == 4, 'step'\n"
            "assert t.call_bwd(lib) == 4, 'backward'\n"
            "assert t.call_conv(lib) == 4, 'conv1d'\n"
            "assert t.call_ssd(lib) == 4, 'ssd'\n"
            "assert lib.ss_status_string(4).startswith(b'SS_ERR_HIP')\n"
            "print('hip failure path ok')\n") % (TESTS, ROOT)
    r = _run([sys.executable, "-c", code], {"SS_SANITIZED_LIB": str(lib), "SS_STUB_LAUNCH_ERROR": "17"})
    assert r.returncode == 0 and "hip failure path ok" in r.stdout, (r.stdout[-2000:], r.stderr[-3000:])
