"""Pins for the stream-K schedule oracle (CPU only).

- hand-derived tables (tests/golden/schedule_cases.json);
- a brute-force construction through a different route: the flattened list
  of (head, tile) pairs is built explicitly and cut with numpy.array_split,
  whose first (I mod G) pieces are one longer -- the same remainder reading;
- invariants: every tile covered once, CTA sizes differ by at most one,
  exactly one host and one finishing segment per head, host_cta/last_cta hold
  the head's first/last tile, at most one partial (non-host segment) per CTA;
- the FlashAttention-2 and FlashDecoding special cases (xllm-io paper review
  of arXiv 2405.10480, §4.3).
"""
from __future__ import annotations

import json
import os
import random

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_schedule(ctx_lens, H, L, G_req):
    T = [-(-n // L) for n in ctx_lens]
    flat = [(b * H + h, t) for b in range(len(T)) for h in range(H) for t in range(T[b])]
    G = min(G_req, len(flat))
    pieces = np.array_split(np.arange(len(flat)), G)
    seg = []
    for c, p in enumerate(pieces):
        run = None
        for i in p:
            u, t = flat[i]
            if run is not None and run[1] == u:
                run[3] = t + 1
            else:
                if run is not None:
                    seg.append(tuple(run))
                run = [c, u, t, t + 1]
        seg.append(tuple(run))
    out = []
    for c, u, t0, t1 in seg:
        Tu = T[u // H]
        out.append((c, u, t0, t1, int(t0 == 0), int(t1 == Tu)))
    owner = {}
    for c, p in enumerate(pieces):
        for i in p:
            owner[flat[i]] = c
    host = [owner[(u, 0)] for u in range(len(T) * H)]
    last = [owner[(u, T[u // H] - 1)] for u in range(len(T) * H)]
    return out, host, last, G


def check_invariants(s, ctx_lens, H, L):
    T = s["T"]
    B = len(ctx_lens)
    G, I = s["G"], s["I"]
    assert I == H * sum(T)
    sizes = np.diff(s["cta_begin"])
    assert s["cta_begin"][0] == 0 and s["cta_begin"][-1] == I
    assert sizes.min() >= 1 and sizes.max() - sizes.min() <= 1
    assert list(sizes) == sorted(sizes, reverse=True)     # the longer CTAs come first
    cover = {}
    hosts = {}
    fins = {}
    for k, (c, u, t0, t1, host, fin) in enumerate(s["seg"]):
        assert s["cta_seg"][c] <= k < s["cta_seg"][c + 1]
        assert 0 <= t0 < t1 <= T[u // H]
        for t in range(t0, t1):
            assert (u, t) not in cover
            cover[(u, t)] = c
        if host:
            assert (u not in hosts) and t0 == 0
            hosts[u] = c
        if fin:
            assert (u not in fins) and t1 == T[u // H]
            fins[u] = c
    assert len(cover) == I
    assert sorted(hosts) == list(range(B * H)) == sorted(fins)
    assert [hosts[u] for u in range(B * H)] == s["host_cta"]
    assert [fins[u] for u in range(B * H)] == s["last_cta"]
    for c in range(G):
        rows = s["seg"][s["cta_seg"][c]:s["cta_seg"][c + 1]]
        assert sum(r[3] - r[2] for r in rows) == sizes[c]
        # only the first segment may be a peer (non-host); only the last may be
        # a host that is not finishing: at most one partial written per CTA
        assert all(r[4] for r in rows[1:])
        assert all(r[5] for r in rows[:-1])
        # the host of a head is its lowest CTA; peers are contiguous after it
        for r in rows:
            u = r[1]
            assert s["host_cta"][u] <= c <= s["last_cta"][u]


def test_golden_tables():
    cases = json.load(open(os.path.join(GOLDEN, "schedule_cases.json")))["cases"]
    for c in cases:
        s = oracle.lean_schedule(c["ctx_lens"], c["H"], c["L"], c["G_req"])
        for key in ("I", "G", "S", "cta_begin", "cta_seg", "host_cta", "last_cta"):
            assert s[key] == c[key], (c["name"], key)
        assert [list(r) for r in s["seg"]] == c["seg"], c["name"]
        check_invariants(s, c["ctx_lens"], c["H"], c["L"])


def _random_cases(n, seed):
    rng = random.Random(seed)
    for _ in range(n):
        B = rng.randint(1, 6)
        H = rng.randint(1, 5)
        L = rng.choice([1, 2, 3, 4, 7, 16])
        lens = [rng.randint(1, 60) for _ in range(B)]
        G = rng.randint(1, 80)
        yield lens, H, L, G


def test_brute_force_and_invariants_random():
    for lens, H, L, G in _random_cases(600, 1):
        s = oracle.lean_schedule(lens, H, L, G)
        seg, host, last, Gb = brute_schedule(lens, H, L, G)
        assert s["G"] == Gb
        assert s["seg"] == seg, (lens, H, L, G)
        assert s["host_cta"] == host and s["last_cta"] == last
        check_invariants(s, lens, H, L)


def test_cta_of_iteration_matches_bounds():
    for I in range(1, 60):
        for G in range(1, I + 1):
            q, r = divmod(I, G)
            bounds = [c * q + min(c, r) for c in range(G + 1)]
            for i in range(I):
                c = oracle.cta_of_iteration(i, I, G)
                assert bounds[c] <= i < bounds[c + 1]


@pytest.mark.parametrize("B,H,T", [(1, 4, 5), (3, 2, 7), (2, 8, 1)])
def test_fa2_special_case(B, H, T):
    """Output tiles = grid size: each CTA computes one whole head."""
    L = 16
    s = oracle.lean_schedule([T * L - 3] * B, H, L, B * H)
    assert s["G"] == B * H
    assert s["seg"] == [(u, u, 0, T, 1, 1) for u in range(B * H)]


@pytest.mark.parametrize("B,H,k,T", [(1, 4, 2, 6), (2, 3, 4, 8), (1, 1, 8, 8)])
def test_fd_special_case(B, H, k, T):
    """Grid an integer multiple k of the output tiles, k | T: every head is
    split into k equal pieces, as a fixed split would."""
    L = 8
    s = oracle.lean_schedule([T * L] * B, H, L, k * B * H)
    assert s["G"] == k * B * H
    w = T // k
    want = []
    for u in range(B * H):
        for j in range(k):
            want.append((u * k + j, u, j * w, (j + 1) * w, int(j == 0), int(j == k - 1)))
    assert s["seg"] == want


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.lean_schedule([4, 0], 2, 4, 3)
    with pytest.raises(ValueError):
        oracle.lean_schedule([4], 2, 0, 3)
    with pytest.raises(ValueError):
        oracle.lean_schedule([4], 0, 4, 3)
    with pytest.raises(ValueError):
        oracle.lean_schedule([4], 1, 4, 0)


def test_pins_catch_planted_mistake():
    """A scheduler that gives the remainder to the last CTAs instead of the
    first fails both the golden tables and the brute force."""
    def bad(ctx_lens, H, L, G_req):
        s = oracle.lean_schedule(ctx_lens, H, L, G_req)
        I, G = s["I"], s["G"]
        q, r = divmod(I, G)
        s["cta_begin"] = [c * q + max(0, c - (G - r)) for c in range(G + 1)]
        return s
    c = json.load(open(os.path.join(GOLDEN, "schedule_cases.json")))["cases"][1]
    assert bad(c["ctx_lens"], c["H"], c["L"], c["G_req"])["cta_begin"] != c["cta_begin"]
