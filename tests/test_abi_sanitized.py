"""The argument checks built for the host alone, under the address and
undefined-behaviour sanitizers.

qmv_api.cpp (every entry point's validation, with the sizes and plans of
qmv_layout.h) is compiled with g++ -fsanitize=address,undefined and linked with
stand-in launchers and no HIP runtime: the link itself shows that validation
reaches no HIP function, and the driver (tests/abi_host/validation_driver.cpp)
runs every entry point through valid calls, every truncated byte size and
extreme counts (INT_MIN .. INT_MAX) with the sanitizers watching. The memra
README's recent-fixes list asks the same of its own input handling: malformed or
truncated input gives a contextual error, never a crash.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gguf_block_quantized_qmv_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "abi_host")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("no host C++ compiler")
    out = str(tmp_path_factory.mktemp("abi_host") / "validation_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-Wall", "-Wextra", "-Werror", "-I" + os.path.join(ROOT, "include"),
           os.path.join(CSRC, "qmv_api.cpp"), os.path.join(HOST, "stub_launchers.cpp"),
           os.path.join(HOST, "validation_driver.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"host-only build failed (a HIP symbol would fail the link):\n{r.stderr}"
    return out


def test_validation_links_without_hip_and_is_sanitizer_clean(driver):
    # verify_asan_link_order=0: the environment may preload libraries of its own ahead of the ASan runtime
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout, r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
