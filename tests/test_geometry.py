"""Host-side bounds check of the balance launches (no GPU).

tests/geometry_check.cpp walks every workgroup and thread of the count, plan
and reroute launches with the kernels' own index functions
(csrc/ultraep_geometry.h) and checks each global index against the buffer
the library sizes for it.  It runs here over the edge shapes of the GPU
parity tests and the eight workloads, one and several layers per call, and
must reject planted index mistakes of the kinds that once faulted the plan
launch on the GPU (a batch of histogram loads without its clamp to the last
tile row; the early local-take loads made for a layer without tokens), and a
reroute block order that is not a bijection when the grid is not a multiple
of eight workgroups.
"""
import os
import shutil
import subprocess

import pytest

import moe_expert_load_ultraep_amd as U

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.dirname(U.LIB_PATH)

pytestmark = pytest.mark.skipif(not os.path.exists(U.LIB_PATH) or shutil.which("hipcc") is None,
                                reason="needs the built library and hipcc")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("geometry") / "geometry_check")
    cmd = ["hipcc", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I",
           os.path.join(PKG, "csrc"), os.path.join(HERE, "geometry_check.cpp"), "-L", PKG, "-lultraep",
           f"-Wl,-rpath,{PKG}", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def run(checker, *args):
    r = subprocess.run([checker, *map(str, args)], capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout + r.stderr


# (E, R, S, D, T, k): the GPU tests' edge shapes and the workloads
SHAPES = [
    (8, 4, 1, 4, 0, 2), (8, 4, 1, 4, 1, 1), (12, 4, 2, 2, 333, 3), (16, 4, 0, 4, 500, 2),
    (16, 4, 2, 1, 500, 2), (32, 8, 3, 4, 2049, 4), (64, 64, 1, 64, 700, 1),
    (1024, 64, 8, 64, 512, 16), (512, 512, 2, 64, 32, 8), (1024, 512, 1, 64, 32, 8),
    (1024, 1024, 1, 64, 16, 8), (512, 512, 1, 8, 32, 8), (160, 40, 3, 8, 1000, 8),
    (3, 3, 2, 3, 3000, 2), (16, 4, 2, 4, 5000, 4), (64, 64, 1, 64, 20000, 1), (4, 2, 2, 2, 3000, 2),
    (64, 4, 1, 4, 1_200_000, 1),
    (8, 4, 1, 4, 256, 2),            # tiny
    (128, 64, 2, 64, 8192, 8),       # single layer / stream
    (256, 64, 2, 64, 4096, 8),       # 61 layers
    (160, 40, 3, 8, 16384, 8),       # topology
    (256, 64, 2, 64, 8192, 8),       # the pages' table shape
    (24, 6, 2, 3, 2000, 8),          # the GPU block-order test: 12 tiles a layer, ragged
]


@pytest.mark.parametrize("E,R,S,D,T,k", SHAPES)
def test_launch_indices_in_bounds(checker, E, R, S, D, T, k):
    for L in (1, 3, 8):
        if L * R * T * k > 200_000_000:
            continue
        rc, out = run(checker, E, R, S, D, L, T, k)
        assert rc == 0, out


def test_deep_workload_all_layers(checker):
    rc, out = run(checker, 256, 64, 2, 64, 61, 4096, 8)
    assert rc == 0, out


@pytest.mark.parametrize("plant,T", [("sum-row", 256), ("scan-row", 256), ("scan-ew", 256),
                                     ("local-first", 0)])
def test_planted_index_mistakes_are_caught(checker, plant, T):
    rc, out = run(checker, 8, 4, 1, 4, 8, T, 2, plant)
    assert rc == 1 and "out of bounds" in out, out


def test_planted_block_order_mistake_is_caught(checker):
    # 3 layers of 4 tiles: 12 reroute workgroups, 4 past the last group of 8
    rc, out = run(checker, 8, 4, 1, 4, 3, 256, 2, "xcd-tail")
    assert rc == 1 and "reroute" in out, out
    rc, out = run(checker, 8, 4, 1, 4, 3, 256, 2)
    assert rc == 0, out
