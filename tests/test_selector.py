"""The shape-driven kind selection (kind="auto"), host only: its grid rule and
its per-head decision checked against the oracle's schedule, which must split
no head when the selection is per-head (xllm-io paper review §4.3: the
stream-K schedule with whole heads per workgroup is the per-head one); grouped
units go per head only when they average at least 4 tiles; short single-head
units that all run at once (K and V of each within 256 KiB, no more heads than
CUs) go per head whatever the schedule."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import decode_phase_attention_amd as la
from oracle.schedule import lean_schedule


def units(H, Hk, Nq):
    cols = H // Hk * Nq
    return H if cols == 1 else Hk * ((cols + 15) // 16)


def expected(lens, H, d, cus, cores, Hk=None, Nq=1, L=None):
    Hk = Hk or H
    U = units(H, Hk, Nq)
    L = L or la.la_default_tile(d)
    tiles = sum((n + L - 1) // L for n in lens)       # one unit of every request
    G = 2 * cus if len(lens) * U >= 2 * cus and tiles < 128 * len(lens) else cus
    G = min(G, cores)
    single = H // Hk * Nq == 1
    if single and len(lens) * U <= cus and max(lens) * 4 * d <= 256 * 1024:
        return "per_head", G            # short heads, all at once: latency-bound
    s = lean_schedule(lens, U, L, G)
    whole = all(h == l for h, l in zip(s["host_cta"], s["last_cta"]))
    long_units = single or s["I"] >= 4 * len(lens) * U
    return ("per_head" if whole and long_units else "lean"), G


@pytest.mark.parametrize("seed", range(40))
def test_matches_oracle_schedule(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 80))
    H, Hk = [(32, 32), (8, 8), (32, 8), (16, 1), (4, 4)][seed % 5]
    Nq = [1, 1, 4, 2, 8][seed % 5]
    d = [128, 64][seed % 2]
    cus = int(rng.choice([8, 32, 104, 256]))
    cores = cus * int(rng.integers(1, 5))
    if seed % 3 == 0:
        lens = [int(rng.integers(8, 5000))] * B              # uniform
    else:
        lens = [int(x) for x in rng.integers(8, 20000, B)]   # ragged
    got = la.la_select_for(lens, H, d, cus, cores, kv_heads=Hk, q_tokens=Nq)
    assert got == expected(lens, H, d, cus, cores, Hk, Nq), (B, H, Hk, Nq, d, cus, cores)


def test_identities_of_the_pages():
    # one long head, few heads: stream-K splits them -> lean on one workgroup per CU
    assert la.la_select_for([524288], 32, 128, 256, 1024) == ("lean", 256)
    # uniform lengths, whole heads per workgroup (B*H = 512 on 512 workgroups): per head
    assert la.la_select_for([4096] * 16, 32, 128, 256, 1024) == ("per_head", 512)
    # ... also when the heads are short (2 tiles each): several per-head
    # workgroups per CU hide the latency of a short head's few steps
    assert la.la_select_for([256] * 512, 8, 128, 256, 1024) == ("per_head", 512)
    assert la.la_select_for([1024] * 512, 8, 128, 256, 1024) == ("per_head", 512)
    # grouped units of 2 tiles stay on lean, of 4 tiles go per head
    assert la.la_select_for([256] * 256, 32, 128, 256, 1024, kv_heads=8) == ("lean", 512)
    assert la.la_select_for([512] * 128, 64, 128, 256, 1024, kv_heads=8) == ("per_head", 512)
    # uniform lengths that do not divide evenly: heads get split -> lean
    assert la.la_select_for([4096] * 9, 32, 128, 256, 1024) == ("lean", 256)
    # ragged batch of many heads: lean on two workgroups per CU ...
    assert la.la_select_for([1000, 3000, 7, 9000] * 4, 32, 128, 256, 1024) == ("lean", 512)
    # ... on one per CU once the heads average 128 tiles or more (mean 237 here)
    assert la.la_select_for([1000, 30000, 7, 90000] * 4, 32, 128, 256, 1024) == ("lean", 256)
    assert la.la_select_for([16129, 16384] * 8, 32, 128, 256, 1024) == ("lean", 512)  # 127.5
    assert la.la_select_for([16129, 16385] * 8, 32, 128, 256, 1024) == ("lean", 256)  # 128
    # the grid never exceeds the co-resident capacity
    assert la.la_select_for([1000, 3000, 7, 9000] * 4, 32, 128, 256, 384)[1] == 384
    # explicit tile size: 64 heads of 5 tiles on 256 workgroups -> split
    assert la.la_select_for([600] * 2, 32, 128, 256, 1024, tile_tokens=128) == ("lean", 256)
    # short heads that all run at once: per head (1024 tokens x 4 x 64 bytes = 256 KiB)
    assert la.la_select_for([1024], 4, 64, 256, 1024) == ("per_head", 256)
    assert la.la_select_for([1025], 4, 64, 256, 1024) == ("lean", 256)
    assert la.la_select_for([512] * 8, 32, 128, 256, 1024) == ("per_head", 256)
    # ... but not when there are more units than CUs
    assert la.la_select_for([512] * 9, 32, 128, 256, 1024) == ("lean", 256)
    # not for grouped heads, whose per-head kernel is slow on short units
    assert la.la_select_for([512] * 8, 32, 128, 256, 1024, kv_heads=8) == ("lean", 256)


def test_validation():
    L = la.lib()
    lens = (ctypes.c_int32 * 2)(16, 16)
    k, g = ctypes.c_int(), ctypes.c_int()
    bad = [
        dict(H=0), dict(d=96), dict(kv_heads=3), dict(q_tokens=65), dict(cus=0),
        dict(coresident=0), dict(tile_tokens=-1),
    ]
    for over in bad:
        a = dict(B=2, H=4, d=128, kv_heads=0, q_tokens=0, tile_tokens=0, cus=8, coresident=8)
        a.update(over)
        st = L.la_select_for(lens, a["B"], a["H"], a["d"], a["kv_heads"], a["q_tokens"],
                             a["tile_tokens"], a["cus"], a["coresident"], ctypes.byref(k),
                             ctypes.byref(g))
        assert st in (1, 2), over
    zero = (ctypes.c_int32 * 2)(16, 0)
    assert L.la_select_for(zero, 2, 4, 128, 0, 0, 0, 8, 8, ctypes.byref(k), ctypes.byref(g)) == 1


def test_auto_rejects_debug_outputs():
    L = la.lib()
    lens = (ctypes.c_int32 * 2)(16, 16)
    fake = 1 << 20
    o = la.binding.LaOpts()
    L.la_opts_init(ctypes.byref(o))
    o.kind = la.LA_KIND_AUTO
    o.tile_owner = fake
    assert L.la_decode_ex(fake, fake, fake, lens, 2, 4, 128, 0.1, fake, None, ctypes.byref(o)) == 1
    o.tile_owner = None
    o.cta_timestamps = fake
    assert L.la_decode_ex(fake, fake, fake, lens, 2, 4, 128, 0.1, fake, None, ctypes.byref(o)) == 1
    assert "explicit kind" in la.la_last_error()
