"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The C ABI's host side: ``hla_api.cpp`` (argument validation, workspace
  sizing, aliasing checks, error text) is built with g++ and both sanitizers
  into a stand-alone library, with the device launchers replaced by stubs
  that abort if reached (``tests/host_sanitize/device_stubs.cpp``); the ABI
  validation tests then run against that library.
* The oracle: a private copy of ``oracle/`` is built with both sanitizers and
  its pin tests run against the copy.

Each run happens in a child process with the sanitizer runtime preloaded and
any report fatal (``-fno-sanitize-recover=all``; leak checking off, since the
Python interpreter itself keeps allocations until exit).  No GPU is involved.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "associative_scan_sequence_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _asan_runtime():
    try:
        path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                              check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


ASAN_RT = _asan_runtime()
pytestmark = pytest.mark.skipif(ASAN_RT is None or shutil.which("g++") is None,
                                reason="gcc's AddressSanitizer runtime is not installed")


def _run_sanitized(args, env_extra=None, timeout=600):
    env = dict(os.environ)
    env.update({"LD_PRELOAD": ASAN_RT, "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",
                "UBSAN_OPTIONS": "print_stacktrace=1"})
    env.update(env_extra or {})
    r = subprocess.run([sys.executable] + args, capture_output=True, text=True, env=env, timeout=timeout)
    text = r.stdout + r.stderr
    assert "runtime error" not in text and "AddressSanitizer" not in text, text[-4000:]
    assert r.returncode == 0, text[-4000:]
    return text


def test_api_validation_under_sanitizers(tmp_path):
    lib = tmp_path / "libhla_host.so"
    subprocess.run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, *SAN, "-fPIC", "-shared", "-o", str(lib),
                    os.path.join(CSRC, "hla_api.cpp"),
                    os.path.join(ROOT, "tests", "host_sanitize", "device_stubs.cpp")],
                   check=True, capture_output=True, text=True)
    runner = tmp_path / "run.py"
    runner.write_text(textwrap.dedent(f'''
        import sys
        sys.path.insert(0, {ROOT!r})
        import associative_scan_sequence_amd._binding as b
        b.load({str(lib)!r})          # every later load() returns this library
        import pytest
        sys.exit(pytest.main(["-q", "-s", "-p", "no:cacheprovider", {os.path.join(ROOT, "tests", "test_abi.py")!r},
                              "-k", "rejects or no_op or status or last_error or noalloc"]))
    '''))
    out = _run_sanitized([str(runner)])
    assert " passed" in out and "failed" not in out, out[-2000:]


def test_oracle_under_sanitizers(tmp_path):
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    for name in os.listdir(os.path.join(ROOT, "oracle")):
        if name.endswith((".py", ".c")):
            shutil.copy(os.path.join(ROOT, "oracle", name), pkg / name)
    # built after the copy, so the loader finds it newer than its sources and keeps it
    subprocess.run(["gcc", "-std=c11", *SAN, "-fPIC", "-shared", "-pthread", "-o", str(pkg / "libhla_oracle.so"),
                    str(pkg / "hla_oracle.c"), str(pkg / "higher_oracle.c")], check=True, capture_output=True,
                   text=True)
    runner = tmp_path / "run.py"
    runner.write_text(textwrap.dedent(f'''
        import sys
        import oracle
        assert oracle.__file__.startswith({str(tmp_path)!r}), oracle.__file__
        import pytest
        sys.exit(pytest.main(["-q", "-s", "-p", "no:cacheprovider",
                              {os.path.join(ROOT, "tests", "test_oracle_pins.py")!r},
                              {os.path.join(ROOT, "tests", "test_higher_oracle.py")!r}]))
    '''))
    # the copy first on the path; the repository next, so the test setup does not put it in front
    out = _run_sanitized([str(runner)], {"PYTHONPATH": f"{tmp_path}{os.pathsep}{ROOT}"})
    assert " passed" in out and "failed" not in out, out[-2000:]
