"""Stress of the in-launch exchange between workgroups (GPU).

Many launches with grids drawn at random -- up to the co-resident maximum, so
a head can have hundreds of peers whose partials its host must see -- each
checked against the fp64 oracle computed once per input. A missing or stale
partial (an ordering bug in the flag/data protocol) shows up as a wrong
output or a raised error word.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def la():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_phase_attention_amd as la
    la.lib()
    return la


CASES = [
    ("bf16", 128, [300000, 3, 50000], 2),
    ("f16", 64, [1, 90000, 777, 4096, 120000], 3),
]


@pytest.mark.parametrize("dtype,d,lens,H", CASES)
def test_random_grids(la, dtype, d, lens, H):
    inp = W.make_custom(lens, H=H, d=d, dtype=dtype, seed=17, device="cuda")
    ref, _, _ = oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), lens,
                                   inp.scale, dtype, workers=8)
    dt = la.LA_BF16 if dtype == "bf16" else la.LA_F16
    cap = la.la_max_grid(d, dt)
    rng = np.random.default_rng(5)
    grids = [cap, cap - 1, 1, 2] + [int(g) for g in rng.integers(1, cap + 1, size=146)]
    tiles = [0, 0, 64, 512] + [int(x) for x in rng.choice([0, 32, 128, 200, 1024], size=146)]
    out = torch.empty((len(lens), H, d), dtype=torch.float32, device="cuda")
    worst = 0.0
    for i, (g, tl) in enumerate(zip(grids, tiles)):
        out.fill_(float("nan"))
        la.la_decode_ex(inp.q, inp.k, inp.v, lens, len(lens), H, d, inp.scale, out, grid=g,
                        tile_tokens=tl, cooperative=(i % 7 == 0))
        la.la_sync_check()
        err = float(np.max(np.abs(out.cpu().numpy() - ref)))
        assert err <= 1e-3, (i, g, tl, err)
        worst = max(worst, err)
    print(f"{dtype} d={d}: {len(grids)} launches, worst max|dO| = {worst:.2e}", file=sys.stderr)


def test_back_to_back_without_sync(la):
    """Launches queued back to back on one stream reuse the flags; each must
    see only its own peers' partials."""
    lens = [200000, 1000]
    H, d = 4, 128
    inp = W.make_custom(lens, H=H, d=d, dtype="bf16", seed=23, device="cuda")
    ref, _, _ = oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), lens,
                                   inp.scale, "bf16", workers=8)
    cap = la.la_max_grid(d, la.LA_BF16)
    outs = [torch.empty((2, H, d), dtype=torch.float32, device="cuda") for _ in range(64)]
    for i, o in enumerate(outs):
        la.la_decode_ex(inp.q, inp.k, inp.v, lens, 2, H, d, inp.scale, o,
                        grid=[cap, 256, cap - 24, 37][i % 4])
    la.la_sync_check()
    for o in outs:
        assert float(np.max(np.abs(o.cpu().numpy() - ref))) <= 1e-3


@pytest.mark.parametrize("host_tables", [False, True])
@pytest.mark.parametrize("Hk,Nq", [(4, 1), (1, 2)])
def test_decode_steps_with_changing_lengths(la, host_tables, Hk, Nq):
    """Decode steps queued back to back, the context lengths different on
    every call (each launch carries its own schedule: prefix sums in its
    arguments, or tables through the staging ring): every step's output
    against the oracle on that step's lengths. Step i reads the first
    H*sum(lens_i) rows of the same K/V buffers as its packed cache."""
    H, d = 4, 128
    base = [3000, 517, 12000, 64]
    steps = 12
    inp = W.make_custom(base, H, d, "bf16", seed=77, device="cuda", kv_heads=Hk, q_tokens=Nq)
    kb, vb, qb = W.to_bits(inp.k), W.to_bits(inp.v), W.to_bits(inp.q)
    outs, all_lens = [], []
    for i in range(steps):
        lens = [max(n - 37 * i - (i % 3), Nq) for n in base]
        out = torch.full(tuple(inp.q.shape), float("nan"), dtype=torch.float32, device="cuda")
        la.la_decode_ex(inp.q, inp.k, inp.v, lens, len(lens), H, d, inp.scale, out,
                        kv_heads=Hk, q_tokens=Nq, host_tables=host_tables)
        outs.append(out)
        all_lens.append(lens)
    la.la_sync_check()
    for i, (lens, out) in enumerate(zip(all_lens, outs)):
        rows = Hk * sum(lens)
        ref = oracle.attend_fp64(qb, kb[:rows], vb[:rows], lens, inp.scale, "bf16", workers=8,
                                 kv_heads=Hk)[0]
        err = float(np.max(np.abs(out.cpu().numpy() - ref)))
        assert err <= 1e-3, (i, lens, err)


def test_two_streams_concurrently(la):
    """Two streams, each with its own workspace (partials, flags, tables),
    running lean launches of different shapes and kernels side by side with no
    synchronisation between them: every output against the oracle. Both grids
    are one workgroup per CU, so the two launches fit on the device together
    (two per CU, within either kernel's occupancy)."""
    a = W.make_custom([5000, 300, 12000], 8, 128, "bf16", seed=6, device="cuda")
    b = W.make_custom([700] * 9, 4, 64, "f16", seed=7, device="cuda", kv_heads=2)
    refs = [oracle.attend_fp64(W.to_bits(x.q), W.to_bits(x.k), W.to_bits(x.v), x.ctx_lens,
                               x.scale, x.dtype, workers=8, kv_heads=x.Hk)[0] for x in (a, b)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    torch.cuda.synchronize()
    for i in range(16):
        for j, (x, s) in enumerate(zip((a, b), streams)):
            with torch.cuda.stream(s):
                out = torch.empty(tuple(x.q.shape), dtype=torch.float32, device="cuda")
                la.la_decode_ex(x.q, x.k, x.v, x.ctx_lens, x.B, x.H, x.d, x.scale, out,
                                kv_heads=x.Hk, host_tables=bool(i % 2))
                outs.append((j, out))
    for s in streams:
        la.la_sync_check(s.cuda_stream)
    torch.cuda.synchronize()
    for j, out in outs:
        err = float(np.max(np.abs(out.cpu().numpy() - refs[j])))
        assert err <= 1e-3, (j, err)


def test_three_streams_past_capacity(la):
    """Three streams, each issuing kind=auto lean launches that pick two
    workgroups per CU: together they ask for more workgroups than the device
    holds at once. The library's budget keeps the unfinished lean launches
    within the co-resident capacity (shrinking a grid, or waiting for another
    stream's launch), so no host waits on a peer that cannot be resident:
    every output meets the oracle and no wait runs out."""
    H, d = 32, 128
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    lens = [int(x) for x in np.random.default_rng(77).integers(2000, 9000, size=16)]
    inp = W.make_custom(lens, H, d, "bf16", seed=77, device="cuda")
    kind, grid = la.la_select(inp.ctx_lens, H, d, la.LA_BF16)
    cap = la.la_max_grid(d, la.LA_BF16)
    say(f"[three streams] auto picks {kind} on {grid} workgroups; capacity {cap}")
    assert kind == "lean" and grid == 2 * cus and 3 * grid > cap
    ref = oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), lens,
                             inp.scale, "bf16", workers=8)[0]
    streams = [torch.cuda.Stream() for _ in range(3)]
    outs = []
    torch.cuda.synchronize()
    for i in range(6):
        for s in streams:
            with torch.cuda.stream(s):
                out = torch.full(tuple(inp.q.shape), float("nan"), dtype=torch.float32,
                                 device="cuda")
                la.la_decode_ex(inp.q, inp.k, inp.v, lens, inp.B, H, d, inp.scale, out,
                                kind="auto")
                outs.append(out)
    for s in streams:
        la.la_sync_check(s.cuda_stream)
    torch.cuda.synchronize()
    for i, out in enumerate(outs):
        err = float(np.max(np.abs(out.cpu().numpy() - ref)))
        assert err <= 1e-3, (i, err)


def _strided(t, lens, Hk, d, S):
    c = torch.full((len(lens), Hk, S, d), float("nan"), dtype=t.dtype, device=t.device)
    row = 0
    for b, n in enumerate(lens):
        c[b, :, :n] = t[row:row + Hk * n].view(Hk, n, d)
        row += Hk * n
    return c


def _random_case(rng):
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["f16", "bf16"]))
    H = int(rng.choice([1, 2, 4, 8, 16, 32]))
    Hk = int(rng.choice([h for h in (1, 2, 4, 8, 16, 32) if H % h == 0]))
    Nq = int(rng.choice([1, 1, 1, 2, 3, 8]))
    B = int(rng.integers(1, 9))
    L = 2048 // d * 8
    lens = []
    for _ in range(B):
        r = rng.random()
        if r < 0.2:
            n = int(rng.integers(1, 4)) * L + int(rng.integers(-1, 2))    # at a tile edge
        else:
            n = int(np.exp(rng.uniform(0, np.log(60000))))
        lens.append(max(n, Nq, 1))
    return d, dtype, H, Hk, Nq, lens


def test_random_shapes_every_kind(la):
    """Random ragged batches, grouped heads, several new tokens, head dims and
    dtypes, packed or capacity-strided caches, under every kind with random
    grids, tiles and chunk sizes; each launch against the oracle on all of
    its query rows."""
    rng = np.random.default_rng(2024)
    kinds = ["lean", "fixed_split", "per_head", "auto", "pull", "chunks"]
    worst = 0.0
    for i in range(60):
        d, dtype, H, Hk, Nq, lens = _random_case(rng)
        kind = kinds[i % len(kinds)]
        grouped = H // Hk * Nq > 1
        opts = {}
        if kind == "lean":
            dt = la.LA_BF16 if dtype == "bf16" else la.LA_F16
            cap = la.la_max_grid_grouped(d, dt) if grouped else la.la_max_grid(d, dt)
            opts = {"grid": int(rng.integers(1, cap + 1)),
                    "tile_tokens": int(rng.choice([0, 16, 64, 300]))}
        elif kind == "fixed_split":
            opts = {"num_splits": int(rng.choice([0, 1, 3, 16, 64]))}
        elif kind == "pull":
            opts = {"grid": int(rng.choice([0, 1, 7, 256, 2000])),
                    "chunk_tiles": int(rng.choice([0, 1, 2, 9]))}
        elif kind == "chunks":
            opts = {"chunk_tiles": int(rng.choice([0, 1, 5, 33]))}
        if (i // 6) % 2 == 1:         # every kind, every other round of six
            opts["kv_stride"] = max(lens) + int(rng.integers(0, 100))
        print(f"[stress {i}] {kind} {opts} d={d} {dtype} H={H} Hk={Hk} Nq={Nq} lens={lens}",
              file=sys.stderr, flush=True)
        inp = W.make_custom(lens, H, d, dtype, seed=100 + i, device="cuda", kv_heads=Hk,
                            q_tokens=Nq)
        ref = oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), lens,
                                 inp.scale, dtype, workers=16, kv_heads=Hk)[0]
        k, v = inp.k, inp.v
        if "kv_stride" in opts:
            # the same rows in a [B, Hk, S, d] cache whose unused rows hold NaN
            k, v = (_strided(t, lens, Hk, d, opts["kv_stride"]) for t in (inp.k, inp.v))
        out = torch.full(tuple(inp.q.shape), float("nan"), dtype=torch.float32, device="cuda")
        la.la_decode_ex(inp.q, k, v, lens, len(lens), H, d, inp.scale, out, kind=kind,
                        kv_heads=Hk, q_tokens=Nq, **opts)
        la.la_sync_check()
        err = float(np.max(np.abs(out.cpu().numpy() - ref)))
        assert err <= 1e-3, (i, kind, opts, err)
        worst = max(worst, err)
    print(f"60 random launches, worst max|dO| = {worst:.2e}", file=sys.stderr)


def test_host_threads_and_shutdown(la):
    """Two host threads, each on its own stream, call the library at once (it
    serialises them internally; error messages are per thread); then
    la_shutdown frees every workspace and later calls build new ones."""
    import threading
    a = W.make_custom([3000, 40], 4, 128, "bf16", seed=31, device="cuda")
    b = W.make_custom([900, 5000, 7], 8, 64, "f16", seed=32, device="cuda", kv_heads=2)
    refs = [oracle.attend_fp64(W.to_bits(x.q), W.to_bits(x.k), W.to_bits(x.v), x.ctx_lens,
                               x.scale, x.dtype, workers=8, kv_heads=x.Hk)[0] for x in (a, b)]
    results, errors = {}, {}

    def worker(j, x):
        s = torch.cuda.Stream()
        outs = []
        with torch.cuda.stream(s):
            for i in range(10):
                out = torch.empty(tuple(x.q.shape), dtype=torch.float32, device="cuda")
                la.la_decode_ex(x.q, x.k, x.v, x.ctx_lens, x.B, x.H, x.d, x.scale, out,
                                kv_heads=x.Hk, kind=["lean", "pull", "fixed_split"][i % 3])
                outs.append(out)
            try:                             # a bad call: its message is this thread's
                la.la_decode_ex(x.q, x.k, x.v, x.ctx_lens, x.B, x.H, x.d, x.scale, outs[0],
                                kv_heads=x.Hk, tile_tokens=-j - 1)
            except la.LaError as e:
                errors[j] = (str(e), la.la_last_error())
            la.la_sync_check(s.cuda_stream)
        results[j] = outs

    threads = [threading.Thread(target=worker, args=(j, x)) for j, x in enumerate((a, b))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    for j in (0, 1):
        for out in results[j]:
            assert float(np.max(np.abs(out.cpu().numpy() - refs[j]))) <= 1e-3, j
        assert "tile_tokens" in errors[j][0] and "tile_tokens" in errors[j][1]
    la.la_shutdown()
    out = torch.empty(tuple(a.q.shape), dtype=torch.float32, device="cuda")
    la.la_decode_ex(a.q, a.k, a.v, a.ctx_lens, a.B, a.H, a.d, a.scale, out)
    la.la_sync_check()
    assert float(np.max(np.abs(out.cpu().numpy() - refs[0]))) <= 1e-3


def _masked_stream(n_cus):
    """A stream whose kernels may use only the first n_cus CUs (default priority)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32,
                                                 ctypes.POINTER(ctypes.c_uint32)]
    total = torch.cuda.get_device_properties(0).multi_processor_count
    words = (total + 31) // 32
    mask = (ctypes.c_uint32 * words)()
    for i in range(n_cus):
        mask[i // 32] |= 1 << (i % 32)
    s = ctypes.c_void_p()
    assert hip.hipExtStreamCreateWithCUMask(ctypes.byref(s), words, mask) == 0
    return torch.cuda.ExternalStream(s.value)


@pytest.mark.parametrize("dtype,d,lens,H", [("bf16", 128, [65536, 65536], 8),
                                            ("f16", 64, [70001, 33333, 9000, 129], 4)])
@pytest.mark.parametrize("n_cus", [100, 200])
def test_crowded_cus(la, dtype, d, lens, H, n_cus):
    """The single-head lean and dynamic pull kernels on a stream confined to
    part of the CUs, so that several of their workgroups share a CU: a wave
    on such a CU finds it crowded (per-CU counters in the control block) and
    switches from K in 16-row blocks to whole rows within a range, on the same
    step grid. Every output meets the oracle, in launches back to back, and a
    launch on the whole device afterwards (counters back at zero) too. Lean
    grids stay within what the masked CUs hold at once, as a lean launch
    needs."""
    inp = W.make_custom(lens, H, d, dtype, seed=d + n_cus, device="cuda")
    ref = oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), lens,
                             inp.scale, dtype, workers=8)[0]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n_cus = min(n_cus, cus)
    per_cu = la.la_max_grid(d, la.LA_BF16 if dtype == "bf16" else la.LA_F16) // cus
    grids = [g for g in (cus, 2 * cus) if g <= per_cu * n_cus]
    assert grids
    st = _masked_stream(n_cus)
    outs = []
    with torch.cuda.stream(st):
        for kind, grid in [("lean", g) for g in grids] + [("pull", 0), ("pull", 2 * cus)]:
            say(f"[crowded] {kind} {dtype} d={d} lens={lens} H={H} cus={n_cus} grid={grid}")
            out = torch.full((len(lens), H, d), float("nan"), dtype=torch.float32, device="cuda")
            la.la_decode_ex(inp.q, inp.k, inp.v, lens, len(lens), H, d, inp.scale, out,
                            kind=kind, grid=grid)
            outs.append(out)
    st.synchronize()
    la.la_sync_check(st.cuda_stream)
    out = torch.full((len(lens), H, d), float("nan"), dtype=torch.float32, device="cuda")
    la.la_decode_ex(inp.q, inp.k, inp.v, lens, len(lens), H, d, inp.scale, out, kind="lean")
    la.la_sync_check()
    outs.append(out)
    for o in outs:
        err = float(np.max(np.abs(o.cpu().numpy() - ref)))
        assert err <= 1e-3, err


@pytest.mark.parametrize("n_cus", [200, 96])
def test_stream_cus(la, n_cus):
    """A stream confined to part of the CUs. Lean's default grid is one
    workgroup per CU of the stream (the executed tile map shows it, and the
    output has the bits of an explicit call at that grid); a grid beyond what
    those CUs hold at once is refused before launch; kind auto takes the pull
    kind for single heads and lean on the stream's CUs for grouped ones, each
    with the bits of the explicit call. Everything meets the oracle. The
    single-head shape gives every workgroup fewer than 8 tiles, so the
    crowding watch is off and the bits cannot depend on where the dispatcher
    put the workgroups (a wave that finds its CU crowded sums its scores in
    another order)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n_cus = min(n_cus, cus - 1)
    st = _masked_stream(n_cus)

    def call(inp, out, stream=None, **o):
        with torch.cuda.stream(stream or torch.cuda.current_stream()):
            la.la_decode_ex(inp.q, inp.k, inp.v, inp.ctx_lens, inp.B, inp.H, inp.d, inp.scale, out,
                            kv_heads=inp.Hk, **o)
        (stream or torch.cuda.current_stream()).synchronize()
        la.la_sync_check((stream or torch.cuda.current_stream()).cuda_stream)
        return out.cpu().numpy()

    def fresh(inp):
        return torch.full((inp.B, inp.H, inp.d), float("nan"), dtype=torch.float32, device="cuda")

    # single heads
    inp = W.make_custom([3000, 17, 6400], 8, 128, "bf16", seed=n_cus, device="cuda")
    ref = oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), inp.ctx_lens,
                             inp.scale, "bf16", workers=8)[0]
    L = la.la_default_tile(128)
    I = inp.H * sum((n + L - 1) // L for n in inp.ctx_lens)
    assert n_cus < I < 8 * n_cus and cus < I < 8 * cus
    say(f"[stream cus] {n_cus} of {cus}: lean default grid, I={I}")
    owner = torch.full((I,), -1, dtype=torch.int32, device="cuda")
    got = call(inp, fresh(inp), st, kind="lean", tile_owner=owner)
    # one workgroup per CU of the stream; single heads on under 70% of the
    # CUs keep the device's default grid (what the stream's CUs hold at most)
    per_cu = la.la_max_grid(128, la.LA_BF16) // cus
    G = n_cus if 10 * n_cus >= 7 * cus else min(la.la_default_grid(128, la.LA_BF16),
                                                 per_cu * n_cus)
    own = owner.cpu().numpy()
    assert own.min() == 0 and own.max() == G - 1 and np.all(np.diff(own) >= 0)
    np.testing.assert_array_equal(got, call(inp, fresh(inp), kind="lean", grid=G))
    assert float(np.max(np.abs(got - ref))) <= 1e-3

    with pytest.raises(la.LaError, match="CUs"):
        call(inp, fresh(inp), st, kind="lean", grid=per_cu * n_cus + 1)
    # the largest grid the stream's CUs hold runs
    assert float(np.max(np.abs(call(inp, fresh(inp), st, kind="lean", grid=per_cu * n_cus) -
                               ref))) <= 1e-3

    say(f"[stream cus] {n_cus}: auto, single heads")
    got = call(inp, fresh(inp), st, kind="auto")
    np.testing.assert_array_equal(got, call(inp, fresh(inp), kind="pull"))
    assert float(np.max(np.abs(got - ref))) <= 1e-3

    # grouped heads: lean on a grid chosen for the stream's CUs
    g = W.make_custom([5000, 900, 33, 20000], 32, 128, "bf16", seed=n_cus + 1, device="cuda",
                      kv_heads=8)
    gref = oracle.attend_fp64(W.to_bits(g.q), W.to_bits(g.k), W.to_bits(g.v), g.ctx_lens,
                              g.scale, "bf16", workers=8, kv_heads=8)[0]
    per_cu_g = la.la_max_grid_grouped(128, la.LA_BF16) // cus
    pick, grid = la.la_select_for(g.ctx_lens, 32, 128, n_cus, per_cu_g * n_cus, kv_heads=8)
    say(f"[stream cus] {n_cus}: auto, grouped -> {pick}@{grid}")
    assert pick == "lean" and grid <= per_cu_g * n_cus
    got = call(g, fresh(g), st, kind="auto")
    np.testing.assert_array_equal(got, call(g, fresh(g), kind="lean", grid=grid))
    assert float(np.max(np.abs(got - gref))) <= 1e-3
