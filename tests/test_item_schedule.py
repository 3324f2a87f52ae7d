"""Host check of the persistent head_dim-128 kernel's work lists (transformer_scaled_dot_amd/csrc/attn_sched.h,
the same source the kernel compiles): every work item is assigned to exactly one workgroup, the head-major
lists keep every head on the XCD of its workgroups, and at the causal 4K shape every workgroup gets the
same number of tile steps."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "transformer_scaled_dot_amd", "csrc")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no g++")
    exe = str(tmp_path_factory.mktemp("sched") / "sched_check")
    subprocess.run([cxx, "-O2", "-std=c++17", "-Wall", "-I" + CSRC, os.path.join(HERE, "sched_check.cpp"), "-o", exe],
                   check=True)
    return exe


def run(exe, G, BH, num_qtiles):
    out = subprocess.run([exe, str(G), str(BH), str(num_qtiles)], check=True, capture_output=True, text=True).stdout
    return {k: int(v) for k, v in (line.split() for line in out.strip().splitlines())}


def grid(BH, num_qtiles, cus=256):
    return min(BH * num_qtiles, cus)


# (BH, query blocks of 256 rows): the causal 4K and 32K shapes, the grouped-heads test shape, small and
# ragged ones, grids that are not whole XCDs
SHAPES = [(64, 16), (32, 128), (16, 16), (8, 3), (6, 3), (3, 1), (1, 1), (40, 7), (64, 2), (128, 1), (24, 24)]


@pytest.mark.parametrize("BH,nq", SHAPES)
def test_every_item_once(checker, BH, nq):
    r = run(checker, grid(BH, nq), BH, nq)
    assert r["bad_index"] == 0
    assert r["assigned_min"] == 1 and r["assigned_max"] == 1


@pytest.mark.parametrize("G", [256, 200, 37])
def test_every_item_once_other_grids(checker, G):
    for BH, nq in SHAPES:
        if BH * nq < G:
            continue
        r = run(checker, G, BH, nq)
        assert r["bad_index"] == 0 and r["assigned_min"] == 1 and r["assigned_max"] == 1, (G, BH, nq)


def test_head_major_keeps_heads_on_their_xcd(checker):
    for BH, nq in [(64, 16), (32, 128), (16, 16), (64, 2)]:
        r = run(checker, grid(BH, nq), BH, nq)
        assert r["by_heads"] == 1, (BH, nq)
        assert r["off_xcd"] == 0, (BH, nq)


def test_head_major_needs_whole_rounds(checker):
    # 6 heads (not a multiple of 8) and 40 heads x 7 blocks on 256 workgroups (35 items per XCD, not a whole
    # number of 32-slot rounds) keep the rotated lists
    assert run(checker, grid(6, 3), 6, 3)["by_heads"] == 0
    assert run(checker, grid(40, 7), 40, 7)["by_heads"] == 0


def test_causal_4k_balance(checker):
    """B4 H16 N4096: 1024 items on 256 workgroups, 136 causal tile steps each."""
    r = run(checker, 256, 64, 16)
    assert r["steps_min"] == r["steps_max"] == 136
