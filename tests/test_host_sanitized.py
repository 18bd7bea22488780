"""The host-side planner (argument checks and workspace layout, plain C++ with
no HIP calls) built with AddressSanitizer and UndefinedBehaviorSanitizer and
driven over ordinary, edge and extreme shapes: no sanitizer report, regions
aligned and in order, and the same codes and sizes as the library reports."""
import ctypes
import os
import random
import shutil
import subprocess

import pytest

from sparse_mixture_experts_prefix_amd import binding as B
from sparse_mixture_experts_prefix_amd import build as native

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(native.PKG, "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("host") / "plan_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(native.ROOT, "include"), "-I", CSRC,
           os.path.join(HERE, "host", "plan_driver.cpp"), os.path.join(CSRC, "plan.cpp"), "-o", out]
    subprocess.run(cmd, check=True)
    return out


def _shapes():
    rng = random.Random(0)
    rows = [
        (4096, 4096, 8, 14336, 2, 0, 0, 0, 0, 0), (64, 2880, 32, 2880, 4, 0, 2, 0, 0, 1),
        (8192, 7168, 256, 2048, 8, 2048, 1, 0, 0, 0), (0, 128, 8, 256, 2, 0, 0, 0, 0, 0),
        (1, 8, 1, 8, 1, 0, 0, 0, 0, 0), (16384, 4096, 8, 14336, 2, 0, 1, 0, 0, 0),
        (700, 512, 64, 256, 8, 256, 0, 16, 16, 0), (5, 128, 8, 256, 2, 64, 0, 0, 0, 1),
        # invalid or unsupported
        (-1, 128, 8, 256, 2, 0, 0, 0, 0, 0), (64, 100, 8, 256, 2, 0, 0, 0, 0, 0),
        (64, 128, 8, 256, 9, 0, 0, 0, 0, 0), (64, 128, 257, 256, 2, 0, 0, 0, 0, 0),
        (64, 128, 8, 256, 2, 0, 3, 0, 0, 0), (64, 128, 8, 256, 2, 0, 0, 6, 3, 0),
        (64, 128, 8, 256, 2, 0, 0, 0, 0, 2), (2 ** 31 - 1, 8, 8, 8, 8, 0, 0, 0, 0, 0),
        (2 ** 20, 2 ** 16, 8, 2 ** 16, 2, 0, 0, 0, 0, 0), (65536, 65536, 256, 65536, 8, 65536, 0, 0, 0, 0),
    ]
    for _ in range(300):
        E = rng.choice([1, 2, 8, 32, 64, 256])
        k = rng.randint(1, min(E, 8))
        rows.append((rng.choice([0, 1, 7, 64, 333, 4096, 70000]), 8 * rng.randint(1, 1024), E,
                     8 * rng.randint(1, 2048), k, rng.choice([0, 0, 8 * rng.randint(1, 512)]),
                     rng.randint(0, 2), 0, 0, rng.randint(0, 1)))
    return rows


def test_planner_under_sanitizers_agrees_with_library(driver):
    rows = _shapes()
    text = "\n".join(" ".join(str(v) for v in r) for r in rows) + "\n"
    res = subprocess.run([driver], input=text, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr
    lines = res.stdout.strip().split("\n")
    assert len(lines) == len(rows)
    lib = B.load_library()
    for r, line in zip(rows, lines):
        vals = [int(v) for v in line.split()]
        shape = B.Shape(*r)
        n = ctypes.c_size_t(0)
        rc = lib.moe_workspace_size(ctypes.byref(shape), ctypes.byref(n))
        assert rc == vals[0], r
        if rc == 0:
            assert vals[1] == lib.moe_block_m(ctypes.byref(shape)) and vals[2] == n.value, r
            rb = lib.moe_backward_workspace_size(ctypes.byref(shape), ctypes.byref(n))
            assert rb == vals[3], r
            if rb == 0:
                assert vals[4] == n.value, r
