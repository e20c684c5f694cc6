"""The lean launch budget across streams (csrc/budget.h), on the host.

A lean launch is correct only if every workgroup its hosts wait for can be
resident. With launches on several streams, the library keeps the unfinished
lean launches of a device within the co-resident capacity (shrinking a new
launch's grid to the room left, or waiting for the oldest other launch when
none is left). The logic is a header-only template over completion events;
this test drives it with fake events."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_phase_attention_amd", "csrc")


def test_budget_logic(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "budget")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-iquote", CSRC,
                    os.path.join(ROOT, "tests", "budget", "budget_main.cpp"), "-o", exe],
                   check=True, capture_output=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
