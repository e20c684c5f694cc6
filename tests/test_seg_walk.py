"""The lean kernels' in-launch segment walk (csrc/seg_walk.h), built on the
host: for every workgroup, the segments it derives from the context lengths
must equal the oracle's stream-K schedule row for row (unit, tile range, host
and finishing flags, the finishing workgroup a host waits for, the linear
iteration of the first tile), plus the request's length and token offset."""
from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.schedule import lean_schedule

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "seg_walk", "walk_main.cpp")
CSRC = os.path.join(ROOT, "decode_phase_attention_amd", "csrc")


@pytest.fixture(scope="module")
def walker(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("walk") / "walk")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-iquote", CSRC, SRC, "-o", exe],
                   check=True, capture_output=True)
    return exe


def walk(exe, lens, U, L, G):
    text = f"{len(lens)} {U} {L} {G} " + " ".join(map(str, lens))
    r = subprocess.run([exe], input=text, capture_output=True, text=True, check=True)
    return [tuple(int(x) for x in line.split()) for line in r.stdout.splitlines()]


def expected(lens, U, L, G_req):
    s = lean_schedule(lens, U, L, G_req)
    tok = np.concatenate([[0], np.cumsum(lens)]).tolist()
    rows = []
    for c, u, t0, t1, host, fin in s["seg"]:
        b = u // U
        last = s["last_cta"][u] if host and not fin else 0
        rows.append((c, u, t0, t1, host, fin, last, s["S"][u] + t0, lens[b], tok[b]))
    return s["G"], rows


CASES = [([1], 1, 256, 1), ([1, 1, 1], 4, 16, 64), ([37, 5, 200, 64], 3, 16, 7),
         ([524288], 32, 256, 256), ([4096] * 16, 32, 256, 512), ([400] * 256, 8, 64, 512),
         # I = 2^31 - 128, just below the 32-bit limit the host enforces
         ([(1 << 24) - 1] * 2, 64, 1, 1023),
         # 255 * (2^24 - 1) tokens: offsets past 2^31 in the 32-bit unsigned prefix
         ([(1 << 24) - 1] * 255, 1, 65536, 300)]


@pytest.mark.parametrize("lens,U,L,G", CASES)
def test_walk_equals_oracle_schedule(walker, lens, U, L, G):
    Gu, rows = expected(lens, U, L, G)
    assert walk(walker, lens, U, L, Gu) == rows


@pytest.mark.parametrize("seed", range(30))
def test_walk_random_shapes(walker, seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 257))
    U = int(rng.choice([1, 2, 4, 8, 32, 64]))
    L = int(rng.choice([1, 7, 16, 64, 128, 256]))
    hi = int(rng.choice([3, 300, 20000]))
    lens = [int(x) for x in rng.integers(1, hi + 1, B)]
    G = int(rng.integers(1, 1100))
    Gu, rows = expected(lens, U, L, G)
    assert walk(walker, lens, U, L, Gu) == rows


def test_grid_larger_than_the_work(walker):
    """A grid of more workgroups than tile iterations: the first I take one
    iteration each, as the oracle's G = min(G_req, I), and the rest are
    empty."""
    lens, U, L = [3, 40, 17], 2, 16
    Gu, rows = expected(lens, U, L, 50)
    assert Gu < 50
    assert walk(walker, lens, U, L, 50) == rows
