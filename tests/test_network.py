"""The register k-selection's networks and WaveTopK, checked on the CPU.

csrc/network.hpp holds the step tables and lane masks that the device code
runs (wave_ops.hpp drives its bitonic steps from them); tests/network_driver.cpp
runs the same tables in a host model of the lane-stride arrays and prints
one line per check.  What is checked ("Billion-scale similarity search with
GPUs", k-selection section):

* depth closed forms: a sort of 2^n elements takes n(n+1)/2 steps, a merge of
  a bitonic sequence of 2^n elements n steps, in the half-cleaner order;
* the 0-1 principle: the 64-element sort (both directions) on every 0-1 input
  of at most three runs and on 200,000 random ones, plus inputs with ties;
  the merges of 64 to 256 elements on every bitonic 0-1 input, of 512 and
  1024 on samples; each output sorted and a permutation of the input pairs;
* the WarpSelect invariants, on a model of WaveTopK fed random streams (ties
  included, k from 1 to 1024): W stays sorted; every one of the k smallest
  values seen so far is in W or the staging buffer; the filter threshold is
  never below the k-th smallest value seen; at the end W holds the k smallest,
  with distinct positions that carry those values.

The driver is also built with three planted mistakes (a schedule step
dropped, one keep-mask bit flipped, the buffer copied over W's last register
instead of the element-wise minimum), and each must make a check fail."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "approximate_nearest_neighbour_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "network_driver.cpp")


def build(tmp_path_factory, name, defines=()):
    exe = str(tmp_path_factory.mktemp("net") / name)
    cmd = ["g++", "-std=c++17", "-O2", "-I", CSRC, *[f"-D{d}" for d in defines], SRC, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip(f"host compiler could not build the network driver: {r.stderr[:300]}")
    return exe


def run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    lines = [l.split() for l in r.stdout.splitlines() if l.strip()]
    return r.returncode, lines


@pytest.fixture(scope="module")
def results(tmp_path_factory):
    return run(build(tmp_path_factory, "network_driver"))


EXPECTED = ["depth_closed_forms", "sort64_asc_zero_one", "sort64_desc_zero_one",
            "merge_bitonic_zero_one_R1", "merge_bitonic_zero_one_R2", "merge_bitonic_zero_one_R4",
            "merge_bitonic_zero_one_R8", "merge_bitonic_zero_one_R16", "topk_nw1_k1",
            "topk_nw1_k10", "topk_nw1_k64", "topk_nw2_k100", "topk_nw2_k128_heavy_ties",
            "topk_nw16_k1000", "topk_nw16_k1024_three_values"]


@pytest.mark.parametrize("name", EXPECTED)
def test_network_check(results, name):
    rc, lines = results
    got = {l[1]: l[0] for l in lines if len(l) >= 2 and l[0] in ("ok", "FAIL")}
    assert got.get(name) == "ok", [l for l in lines if len(l) > 1 and l[1] == name]


def test_driver_exit_status(results):
    rc, lines = results
    assert rc == 0 and lines[-1] == ["done", "0"]


@pytest.mark.parametrize("plant,expect", [
    ("PLANT_SKIP_STEP", "sort64_asc_zero_one"),
    ("PLANT_MASK_BIT", "sort64_asc_zero_one"),
    ("PLANT_NO_FOLD", "topk_nw1_k10"),
])
def test_planted_mistake_is_caught(tmp_path_factory, plant, expect):
    rc, lines = run(build(tmp_path_factory, plant.lower(), [plant]))
    failed = {l[1] for l in lines if len(l) >= 2 and l[0] == "FAIL"}
    assert rc != 0 and expect in failed, failed
