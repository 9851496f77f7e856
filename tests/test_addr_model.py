"""Every weight load of every kernel, checked on the host.

The kernels form their weight addresses with the functions of
gguf_block_quantized_qmv_amd/csrc/qmv_addr.h (launch plans, per-lane bases,
step and unit offsets, read windows). tests/abi_host/addr_model.cpp runs those
same functions, built with g++ under the address and undefined-behaviour
sanitizers, over every lane of the workgroups each launch runs (all of them for
small grids, the first and last three otherwise), every step and unit the
kernels issue, for the instantiations the entry points choose over a sweep of
shapes: each dense-GEMV row length up to 18432 and the runtime loop beyond, row
counts that take each workgroup shape, M = 1..4, the Q4_K and IQ4_XS routed
experts of the 35B-A3B layer (memra README speed table) and ragged ones, the
grouped prefill and the K-split prefill GEMM. Every read must lie inside the
weights, and every read whose data is used inside the lane's own row.

The same driver with the dense GEMV's earlier step rule (every step below the
row's step count taken as the lane's own, the partial last step included) must
find the over-read that rule had at K = 17408: up to 576 bytes past the end of
the weights, from the last row's lanes past the half-used last step.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "abi_host")

ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("no host C++ compiler")
    out = str(tmp_path_factory.mktemp("addr_model") / "addr_model")
    cmd = ["g++", "-std=c++17", "-O2", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-Wall", "-Wextra", "-Werror", "-I" + os.path.join(ROOT, "include"),
           os.path.join(HOST, "addr_model.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def test_every_weight_load_in_bounds(model):
    r = subprocess.run([model], capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "0 past the weights, 0 used reads outside their row, 0 other violations" in r.stdout, r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr


def test_earlier_step_rule_is_caught(model):
    r = subprocess.run([model, "--prefix"], capture_output=True, text=True, env=ENV, timeout=120)
    assert r.returncode == 3, r.stdout + r.stderr
    assert "up to 576 bytes past the end" in r.stdout, r.stdout
    assert "k 17408" in r.stdout, r.stdout
