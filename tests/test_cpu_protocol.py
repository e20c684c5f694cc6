"""CPU emulation of the kernels' cross-workgroup exchange (tests/cpu_protocol).

One thread per workgroup runs the real stream-K tables from the library's host
scheduler (lean) or pulls chunks from a counter (pull), in fp64 with random
delays, under ThreadSanitizer. The merged outputs must equal the fp64 oracle,
the pull results must be bitwise the same for any thread count and timing, no
counter may be left raised, TSan must report nothing, and a peer that never
raises its flag must end in an error, not a hang (the watchdog path). Lean
launches run back to back on one exchange: a peer that raises its flag late
in one launch (after its host gave up) must not disturb the next ones, and
the earlier protocol without epochs must be caught doing exactly that."""
from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import oracle
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "cpu_protocol", "emulator.cpp")
CSRC = os.path.join(ROOT, "decode_phase_attention_amd", "csrc")


def build(tmp_path_factory, name, *defines):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("emu") / name)
    # host code only: g++ with ThreadSanitizer
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=thread", *defines, "-iquote", CSRC, SRC,
           os.path.join(CSRC, "sched.cpp"), "-o", exe, "-lpthread"]
    subprocess.run(cmd, check=True, capture_output=True)
    return exe


@pytest.fixture(scope="module")
def emulator(tmp_path_factory):
    return build(tmp_path_factory, "emu_tsan")


def problem(lens, H, d, seed):
    inp = W.make_custom(lens, H, d, "f16", seed=seed)
    f64 = lambda t: t.to(torch.float64).numpy()
    return inp, f64(inp.q), f64(inp.k), f64(inp.v)


def run(emulator, tmp_path, inp, q, k, v, mode, G, C=0, drop=-1, wait_ms=5000, seed=1, L=8,
        launches=1, expect_race=False):
    B, H, d = inp.B, inp.H, inp.d
    hdr = np.array([mode, B, H, d, L, G, C, drop, wait_ms, seed, launches], np.int32)
    fin, fout = tmp_path / f"in_{mode}_{G}_{C}_{seed}", tmp_path / f"out_{mode}_{G}_{C}_{seed}"
    with open(fin, "wb") as f:
        f.write(hdr.tobytes())
        f.write(np.array(inp.ctx_lens, np.int32).tobytes())
        f.write(np.array([inp.scale], np.float64).tobytes())
        for a in (q, k, v):
            f.write(np.ascontiguousarray(a, np.float64).tobytes())
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 exitcode=66")
    r = subprocess.run([emulator, str(fin), str(fout)], capture_output=True, text=True, env=env,
                       timeout=120)
    if expect_race:
        return r
    assert r.returncode == 0, r.stderr[-3000:]
    assert "ThreadSanitizer" not in r.stderr, r.stderr[-3000:]
    raw = open(fout, "rb").read()
    st = int(np.frombuffer(raw[:4], np.int32)[0])
    vals = np.frombuffer(raw[4:], np.float64)
    n = B * H
    return st, vals[:n * d].reshape(B, H, d), vals[n * d:n * d + n].reshape(B, H), \
        vals[n * d + n:].reshape(B, H)


def reference(inp):
    return oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), inp.ctx_lens,
                              inp.scale, inp.dtype, workers=1)


def close(got, ref):
    O, m, l = got
    Or, mr, lr = ref
    np.testing.assert_allclose(O, Or, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(m, mr, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l, lr, rtol=1e-10)


CASES = [([37, 5, 200, 64], 3, 16), ([1, 1, 1], 2, 8), ([400], 4, 16)]


@pytest.mark.parametrize("lens,H,d", CASES)
@pytest.mark.parametrize("G", [1, 3, 7, 64])
def test_lean_protocol_equals_oracle(emulator, tmp_path, lens, H, d, G):
    inp, q, k, v = problem(lens, H, d, seed=G)
    st, O, m, l = run(emulator, tmp_path, inp, q, k, v, mode=0, G=G, seed=G)
    assert st == 0
    close((O, m, l), reference(inp))


@pytest.mark.parametrize("lens,H,d", CASES)
@pytest.mark.parametrize("threads,C", [(1, 1), (4, 3), (16, 1), (9, 40)])
def test_pull_protocol_equals_oracle_and_is_bitwise_stable(emulator, tmp_path, lens, H, d,
                                                          threads, C):
    inp, q, k, v = problem(lens, H, d, seed=threads + C)
    st, O, m, l = run(emulator, tmp_path, inp, q, k, v, mode=1, G=threads, C=C, seed=1)
    assert st == 0
    close((O, m, l), reference(inp))
    # another thread count and other delays: the merge tree is fixed, so the
    # bits are the same
    st2, O2, m2, l2 = run(emulator, tmp_path, inp, q, k, v, mode=1, G=threads + 5, C=C, seed=2)
    assert st2 == 0
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(l, l2)


def test_head_over_many_chunk_groups(emulator, tmp_path):
    """One head of 300 one-tile chunks: 19 groups of 16, a last group of 12."""
    inp, q, k, v = problem([2400], 1, 8, seed=5)
    st, O, m, l = run(emulator, tmp_path, inp, q, k, v, mode=1, G=12, C=1, seed=3)
    assert st == 0
    close((O, m, l), reference(inp))


def test_missing_peer_ends_in_error_not_hang(emulator, tmp_path):
    """A peer that never raises its flag: the host's bounded wait gives up."""
    inp, q, k, v = problem([400], 2, 8, seed=6)
    st, O, _, _ = run(emulator, tmp_path, inp, q, k, v, mode=0, G=8, drop=3, wait_ms=200)
    assert st == 4


def test_late_peer_stays_in_its_launch(emulator, tmp_path):
    """Workgroup 3 (a peer of head 0) raises its flag only after its host gave
    up in the first launch, then on time in the next two, with nothing reset
    in between: the sticky error is reported, and the last launch equals the
    oracle on every head."""
    inp, q, k, v = problem([400], 2, 8, seed=6)
    st, O, m, l = run(emulator, tmp_path, inp, q, k, v, mode=0, G=8, drop=3, wait_ms=200,
                      launches=3)
    assert st == 4
    close((O, m, l), reference(inp))


@pytest.mark.parametrize("G", [5, 64])
def test_launches_in_a_row_advance_the_epoch(emulator, tmp_path, G):
    inp, q, k, v = problem([37, 5, 200, 64], 3, 16, seed=G)
    st, O, m, l = run(emulator, tmp_path, inp, q, k, v, mode=0, G=G, seed=G, launches=4)
    assert st == 0      # also: exit count back at zero, epoch == launches
    close((O, m, l), reference(inp))


def test_protocol_without_epochs_is_caught(tmp_path_factory, tmp_path):
    """Plant the earlier protocol (flags 1/0, sticky give-up). After the late
    peer of the first launch, a later launch fails in one of two ways,
    depending on timing. A host sees the stale raised flag and reads the record
    while its peer is still writing it (TSan reports a data race). Or a host
    gives up at once on a peer not yet done, because the error of the first
    launch is sticky, and its heads come out undefined (NaN here). Either is
    caught; the epoch protocol above does neither."""
    bad = build(tmp_path_factory, "emu_unepoched", "-DEMU_UNEPOCHED")
    inp, q, k, v = problem([400], 2, 8, seed=6)
    r = run(bad, tmp_path, inp, q, k, v, mode=0, G=8, drop=3, wait_ms=200, launches=3,
            expect_race=True)
    if r.returncode == 66:
        assert "data race" in r.stderr, r.stderr[-2000:]
        return
    assert r.returncode == 0, r.stderr[-2000:]
    raw = open(tmp_path / "out_0_8_0_1", "rb").read()
    O = np.frombuffer(raw[4:], np.float64)[:inp.B * inp.H * inp.d].reshape(inp.B, inp.H, inp.d)
    Or, _, _ = reference(inp)
    assert not np.allclose(O, Or, rtol=1e-10, atol=1e-12), "the earlier protocol went unnoticed"


@pytest.mark.parametrize("mode,G,C", [(0, 6, 0), (1, 6, 1)])
def test_tsan_catches_unordered_publish(tmp_path_factory, tmp_path, mode, G, C):
    """Plant the mistake (flags and counters without release/acquire): TSan
    must report the race on the records, so a clean run above means
    something."""
    bad = build(tmp_path_factory, "emu_unordered", "-DEMU_UNORDERED_PUBLISH")
    inp, q, k, v = problem([300, 90], 2, 8, seed=7)
    r = run(bad, tmp_path, inp, q, k, v, mode=mode, G=G, C=C, expect_race=True)
    assert r.returncode == 66 and "data race" in r.stderr, (r.returncode, r.stderr[-2000:])
