"""The attention kernel's work order, checked on the host: work_order.h is
compiled as plain host code (hipcc, no GPU needed) into a small program that
walks every queue slot of a layer and checks that the slots cover each
(query-block pair, query head) exactly once, in range and in its KV group.
Shapes: both item orders (pair-major up to 16384 tokens, head-major beyond),
the switch between them, ragged lengths, one block, G = 1, MQA and KV-head
counts below, equal to and above the eight XCDs."""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dynamic_sparse_attention_map_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.environ.get("HIPCC", os.path.join(ROCM, "bin", "hipcc"))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("work_order") / "work_order_check")
    src = os.path.join(ROOT, "tests", "work_order_check.cpp")
    r = subprocess.run([HIPCC if os.path.exists(HIPCC) else "hipcc", "-x", "c++", "-std=c++17", "-O1",
                        "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
                        "-I", CSRC, "-I", os.path.join(ROOT, "include"), src, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return exe


def run(exe, shapes):
    args = [str(x) for s in shapes for x in s]
    r = subprocess.run([exe, *args], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    assert f"{len(shapes)} shapes, 0 failures" in r.stdout


def test_named_shapes(checker):
    run(checker, [
        (1, 2, 1), (128, 4, 4), (379, 3, 3), (2048, 32, 8), (4096, 4, 1), (8192, 32, 8),
        (8192, 28, 4), (12000, 6, 3), (13005, 4, 2), (16384, 32, 8), (16384, 64, 1),
        (16385, 32, 8), (20000, 64, 1), (32768, 32, 8), (40000, 4, 1), (65536, 32, 8),
        (100000, 6, 3), (131072, 32, 8), (131072, 28, 4), (131072, 16, 16), (524288, 32, 8),
    ])


def test_random_shapes(checker):
    rng = np.random.default_rng(20261203)
    shapes = []
    for _ in range(200):
        hkv = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16]))
        hq = hkv * int(rng.choice([1, 2, 3, 4, 7, 8]))
        n = int(rng.integers(1, 70000))
        shapes.append((n, hq, hkv))
    run(checker, shapes)
