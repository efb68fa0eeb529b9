"""Host builds with AddressSanitizer and UndefinedBehaviorSanitizer (no GPU): the oracle driven over every
entry point and edge case (tests/sanitize/oracle_check.c, built with gcc), and the host side of the C ABI --
plan choice, host scheduler, workspace sizes and the argument checks of every entry point -- built with
the sanitizers on its host code only (tests/sanitize/api_check.cpp linked against the library sources).
Any sanitizer report fails the test."""
import os
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "sliding_window_decode_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    text = r.stdout + r.stderr
    assert "AddressSanitizer" not in text and "runtime error" not in text, text[-4000:]
    assert r.returncode == 0, text[-4000:]
    return text


def test_oracle_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_check")
        subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        "-fno-omit-frame-pointer", "-pthread", os.path.join(HERE, "sanitize", "oracle_check.c"),
                        os.path.join(ROOT, "oracle", "oracle.c"), "-o", exe, "-lm"], check=True)
        assert "oracle sanitizer check: ok" in _run(exe)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_api_under_asan_and_ubsan():
    srcs = ["sda_api.cpp", "sda_decode_ring.hip", "sda_decode_wide.hip", "sda_decode_staged.hip", "sda_sched.hip",
            "sda_v41.hip"]
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "api_check")
        # the sanitizers instrument the host code only (-Xarch_host), the device code builds as usual
        flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-Xarch_host", "-fsanitize=address",
                 "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all",
                 "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
        objs = []
        for s in srcs + [os.path.join(HERE, "sanitize", "api_check.cpp")]:
            path = s if os.path.isabs(s) else os.path.join(CSRC, s)
            obj = os.path.join(d, os.path.basename(s) + ".o")
            lang = ["-x", "hip"] if path.endswith(".cpp") and "api_check" not in path else []
            subprocess.run([HIPCC, *flags, *lang, "-c", path, "-o", obj], check=True, capture_output=True)
            objs.append(obj)
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                        "-fsanitize=undefined", *objs, "-o", exe], check=True, capture_output=True)
        assert "api sanitizer check: ok" in _run(exe)
