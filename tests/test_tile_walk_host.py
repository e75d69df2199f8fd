"""CPU bounds check of the grouped GEMMs' tile walk.

The index math that maps a workgroup to its tile (XCD-aware one-tile grids, the persistent walk,
the workspace bounds on M-tiles and 256-row tiles) lives in one header that the kernels and
``tests/native/tile_walk_check.cpp`` both include.  The program is built here with address and
undefined-behaviour sanitisers and run over routings of the layer's shapes: uniform, Zipf-like and
one-expert-heavy picks, empty experts, one token, no tokens, and the load vectors that need the most
padded M-tiles and the most 256-row tiles (those meet the planned bounds exactly).  It checks that
every tile is yielded exactly once and inside its segment and the workspace.  Planting a mistake
in the walk (a dropped min, an off-by-one in the XCD deal or a bound) fails it.
"""

import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
SRC = ROOT / "tests" / "native" / "tile_walk_check.cpp"

# T tokens, N routed experts, K picks, Ns shared experts, seed, skew
# (0 uniform, 1 Zipf-like, 2 one favoured expert, 3 loads of 128 q + 1, 4 loads of 256 q + 1)
CASES = [
    (8192, 256, 8, 1, 0, 0),   # prefill shape, uniform picks
    (8192, 256, 8, 1, 1, 1),   # prefill shape, Zipf-like picks: many light experts
    (8192, 256, 8, 1, 0, 3),   # prefill shape, every M-tile bound reached
    (256, 256, 8, 1, 2, 0),    # decode shape: most experts hold a few rows
    (260, 16, 4, 1, 0, 4),     # every segment an odd number of M-tiles: the 256-row bound reached
    (513, 64, 6, 2, 4, 2),     # ragged T, two shared experts, one expert takes every token
    (2048, 512, 32, 1, 5, 3),  # the largest expert count and top-K
    (1, 16, 4, 1, 1, 0),       # one token: twelve empty experts
    (0, 8, 2, 1, 1, 0),        # no tokens
]


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = tmp_path_factory.mktemp("tile_walk") / "tile_walk_check"
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-D_GLIBCXX_ASSERTIONS", "-o", str(exe), str(SRC)], check=True)
    return exe


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T%d_N%d_K%d_Ns%d_s%d_skew%d" % c)
def test_tile_walk_in_bounds(checker, case):
    r = subprocess.run([str(checker)] + [str(v) for v in case], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok:"), r.stdout
    if case[5] == 3:
        # the padded layout meets the planned M-tile bound exactly
        tiles, of = r.stdout.split("tiles=")[1].split()[0:3:2]
        assert tiles == of, r.stdout
    if case[5] == 4:
        pairs, of = r.stdout.split("pairs=")[1].split()[0:3:2]
        assert pairs == of, r.stdout
