"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds a copy of libprope.so whose host code (argument checks, launch set-up,
integer helpers) is instrumented, then reruns the C-ABI tests against it in a
child process with the ASan runtime preloaded, and runs the host integer
checks built with the same sanitizers. Any sanitizer report aborts the child
and fails the test. GPU code is built as usual and never runs here.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "position_remapped_rope_amd", "csrc")
sys.path.insert(0, ROOT)

pytestmark = [pytest.mark.slow,
              pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                 reason="hipcc not available")]

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    from position_remapped_rope_amd import build as b
    try:
        rt = b.asan_runtime()
    except RuntimeError:
        pytest.skip("clang ASan runtime not found")
    out = str(tmp_path_factory.mktemp("asan") / "libprope_asan.so")
    b.build(sanitize_out=out)
    return out, rt


def test_abi_under_asan_ubsan(sanitized_lib):
    lib, rt = sanitized_lib
    env = dict(os.environ, PROPE_LIB_PATH=lib, LD_PRELOAD=rt, **SAN_ENV)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "Sanitizer" not in r.stdout + r.stderr, tail
    assert " passed" in r.stdout, tail


def test_sanitized_library_catches_a_planted_overflow(sanitized_lib):
    """The instrumentation is live: a signed overflow in a scratch host program
    built with the same flags is reported and aborts."""
    lib, rt = sanitized_lib
    from position_remapped_rope_amd import build as b
    tmp = os.path.dirname(lib)
    src = os.path.join(tmp, "planted.cpp")
    with open(src, "w") as f:
        f.write("#include <cstdint>\n#include <cstdio>\nint main(int argc, char**) {\n"
                "  int64_t L = INT64_MAX - 1 + argc;\n  int64_t g = (L + 1) / 2;\n"
                "  std::printf(\"%lld\\n\", (long long)g);\n  return 0;\n}\n")
    exe = os.path.join(tmp, "planted")
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    r = subprocess.run([hipcc, *b.SANITIZE_FLAGS, "-O1", src, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([exe], capture_output=True, text=True, env=dict(os.environ, **SAN_ENV))
    assert out.returncode != 0 and "runtime error" in out.stderr


def test_host_integer_checks_under_asan_ubsan(tmp_path):
    from position_remapped_rope_amd import build as b
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    exe = tmp_path / "fastdiv_check_san"
    r = subprocess.run([hipcc, "-O1", "-std=c++17", "-x", "hip", "--offload-arch=gfx950", *b.SANITIZE_FLAGS,
                        f"-I{CSRC}", os.path.join(ROOT, "tests", "host", "fastdiv_check.cpp"), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=dict(os.environ, **SAN_ENV))
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok ") and "runtime error" not in out.stderr
