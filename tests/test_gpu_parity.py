"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar: max |O_gpu - O_ref| <= 1e-3 on the fp32 output; l within 1e-5 relative
after rescaling to the oracle's max (l_gpu * exp(m_gpu - m_ref) vs l_ref) and
|m_gpu - m_ref| <= 1e-5 * max(1, |m_ref|). The lean kernel's executed
tile-to-workgroup map must equal the schedule oracle's bit for bit.
"""
from __future__ import annotations

import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from fullsize_ref import full_reference

pytestmark = pytest.mark.gpu

O_TOL = 1e-3
L_RTOL = 1e-5
M_RTOL = 1e-5
WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def la():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_phase_attention_amd as la
    la.lib()
    return la


def run(la, inp, kind="lean", **opts):
    B, H, d = inp.B, inp.H, inp.d
    dev = inp.q.device
    out = torch.full((B, H, d), float("nan"), dtype=torch.float32, device=dev)
    m = torch.full((B * H,), float("nan"), dtype=torch.float32, device=dev)
    l = torch.full((B * H,), float("nan"), dtype=torch.float32, device=dev)
    la.la_decode_ex(inp.q, inp.k, inp.v, inp.ctx_lens, B, H, d, inp.scale, out, kind=kind,
                    m_out=m, l_out=l, **opts)
    la.la_sync_check()
    return out.cpu().numpy(), m.view(B, H).cpu().numpy(), l.view(B, H).cpu().numpy()


def reference(inp, heads=None):
    return oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), inp.ctx_lens,
                              inp.scale, inp.dtype, heads=heads, workers=WORKERS)


def reference_kv(inp):
    """The oracle with the inputs' own K/V head count (grouped or not)."""
    return oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), inp.ctx_lens,
                              inp.scale, inp.dtype, workers=WORKERS, kv_heads=inp.Hk)


def sampled_reference(inp, heads):
    """Oracle on a subset of heads, copying only those heads' rows to the host."""
    B, H, d = inp.B, inp.H, inp.d
    starts = np.concatenate([[0], np.cumsum(inp.ctx_lens)]) * H
    qb = W.to_bits(inp.q)
    O = np.full((B, H, d), np.nan)
    M = np.full((B, H), np.nan)
    L = np.full((B, H), np.nan)
    for (b, h) in heads:
        n = inp.ctx_lens[b]
        r0 = int(starts[b]) + h * n
        kb = W.to_bits(inp.k[r0:r0 + n])
        vb = W.to_bits(inp.v[r0:r0 + n])
        o, m, l = oracle.attend_fp64(qb[b:b + 1, h:h + 1], kb, vb, [n], inp.scale, inp.dtype,
                                     workers=1)
        O[b, h], M[b, h], L[b, h] = o[0, 0], m[0, 0], l[0, 0]
    return O, M, L


def check(got, ref, heads=None, tag=""):
    O, m, l = got
    Or, mr, lr = ref
    if heads is not None:
        idx = tuple(np.array(heads).T)
        O, m, l, Or, mr, lr = O[idx], m[idx], l[idx], Or[idx], mr[idx], lr[idx]
    assert np.isfinite(O).all(), tag
    err = float(np.max(np.abs(O - Or)))
    assert err <= O_TOL, f"{tag}: max |dO| = {err}"
    assert np.all(np.abs(m - mr) <= M_RTOL * np.maximum(1.0, np.abs(mr))), f"{tag}: m"
    lrel = np.abs(l * np.exp(m.astype(np.float64) - mr) - lr) / lr
    assert float(np.max(lrel)) <= L_RTOL, f"{tag}: l rel err {float(np.max(lrel))}"
    return err


def tile_owner_ref(lens, H, L, G):
    s = oracle.lean_schedule(lens, H, L, G)
    own = np.empty(s["I"], np.int32)
    for (c, u, t0, t1, _h, _f) in s["seg"]:
        own[s["S"][u] + t0:s["S"][u] + t1] = c
    return own, s["G"]


# ------------------------------------------------------------------ small shapes

KINDS = ["lean", "fixed_split", "per_head"]


@pytest.mark.parametrize("kind", KINDS)
def test_tiny_config(la, kind):
    inp = W.make_inputs("tiny", seed=0, device="cuda")
    say(f"[tiny/{kind}]")
    check(run(la, inp, kind), reference(inp), tag=f"tiny/{kind}")


@pytest.mark.parametrize("dtype,d", [("f16", 64), ("bf16", 64), ("f16", 128), ("bf16", 128)])
@pytest.mark.parametrize("kind", KINDS)
def test_ragged_small(la, dtype, d, kind):
    lens = [1, 7, 129, 1000, 4097, 300]
    inp = W.make_custom(lens, H=3, d=d, dtype=dtype, seed=11, device="cuda")
    say(f"[ragged-small {dtype} d={d} {kind}]")
    ref = reference(inp)
    check(run(la, inp, kind), ref, tag=f"{dtype}/{d}/{kind}")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
def test_step_grid_phase(la, dtype, d):
    """Every range of 8 steps or more starts its step grid at the 4 KiB
    boundary of the K rows at or before its first row and masks the rows of
    the first step that precede it. Caches placed at every row offset within
    4 KiB, with tiles and grids that start long and short ranges at many
    rows, must give the oracle's result on every kind: a row counted twice or
    dropped at a range start shows in l and O."""
    lens = [3, 130, 5000, 77, 2100]
    H = 3
    inp = W.make_custom(lens, H=H, d=d, dtype=dtype, seed=89, device="cuda")
    ref = reference(inp)
    rows = 4096 // (2 * d)
    for r in range(rows):
        kb = torch.zeros((inp.k.shape[0] + r, d), dtype=inp.k.dtype, device="cuda")
        vb = torch.zeros_like(kb)
        kb[r:].copy_(inp.k)
        vb[r:].copy_(inp.v)
        k, v = kb[r:], vb[r:]
        assert k.is_contiguous() and (k.data_ptr() - kb.data_ptr()) == r * 2 * d
        view = W.Inputs(q=inp.q, k=k, v=v, ctx_lens=lens, H=H, d=d, dtype=dtype,
                        scale=inp.scale, seed=89)
        # ranges of 8 and more steps (16-row K blocks, edge steps at every
        # phase) and shorter ones (whole rows)
        for kind, opts in (("lean", {"tile_tokens": 48, "grid": 37}),
                           ("lean", {"tile_tokens": 48, "grid": 3}), ("lean", {"grid": 5}),
                           ("lean", {"tile_tokens": 16, "grid": 5}), ("lean", {}),
                           ("fixed_split", {"num_splits": 3}), ("fixed_split", {"num_splits": 1}),
                           ("per_head", {}), ("pull", {"grid": 7})):
            say(f"[phase {dtype} d={d} offset={r} rows {kind} {opts}]")
            check(run(la, view, kind, **opts), ref, tag=f"d={d}/offset={r}/{kind}/{opts}")


@pytest.mark.parametrize("host_tables", [False, True])
@pytest.mark.parametrize("grid", [1, 2, 3, 7, 255, 0, -1])
@pytest.mark.parametrize("tile", [0, 16, 100, 384])
def test_lean_schedule_invariance(la, grid, tile, host_tables):
    """Any grid (0: the default, -1: the co-resident maximum) and LeanTile size
    gives the oracle's result, and the kernel executes exactly the oracle's
    tile-to-workgroup map, with the segments derived in the launch or read
    from the host's tables."""
    lens = [33, 1, 700, 2048, 5]
    H, d = 4, 128
    inp = W.make_custom(lens, H=H, d=d, dtype="bf16", seed=3, device="cuda")
    L = tile if tile else la.la_default_tile(d)
    if grid == -1:
        grid = la.la_max_grid(d, la.LA_BF16)
    G_req = grid if grid else la.la_default_grid(d, la.LA_BF16)
    own_ref, G = tile_owner_ref(lens, H, L, G_req)
    owner = torch.full((own_ref.size,), -1, dtype=torch.int32, device="cuda")
    say(f"[invariance grid={grid} tile={tile} host_tables={host_tables}]")
    got = run(la, inp, "lean", grid=grid, tile_tokens=tile, tile_owner=owner,
              host_tables=host_tables)
    check(got, reference(inp), tag=f"grid={grid} tile={tile}")
    assert np.array_equal(owner.cpu().numpy(), own_ref)


@pytest.mark.parametrize("splits", [1, 2, 3, 16, 64])
def test_fixed_split_counts(la, splits):
    lens = [3, 1000, 40000]
    inp = W.make_custom(lens, H=2, d=64, dtype="f16", seed=5, device="cuda")
    check(run(la, inp, "fixed_split", num_splits=splits), reference(inp), tag=f"splits={splits}")


@pytest.mark.parametrize("grid", [0, -1])
def test_cooperative_launch(la, grid):
    lens = [5000, 17, 60000]
    inp = W.make_custom(lens, H=8, d=128, dtype="bf16", seed=9, device="cuda")
    g = la.la_max_grid(128, la.LA_BF16) if grid == -1 else 0
    check(run(la, inp, "lean", cooperative=True, grid=g), reference(inp), tag="cooperative")


def test_adversarial_scores(la):
    """Scores spread over tens of units (q scaled up) in fp16 and bf16."""
    for dtype in ("f16", "bf16"):
        inp = W.make_custom([3000, 20000], H=4, d=128, dtype=dtype, seed=21, device="cuda",
                            q_std=6.0)
        got = run(la, inp, "lean", grid=37)
        check(got, reference(inp), tag=f"adversarial/{dtype}")


# ------------------------------------------------------------------ closed forms

def _inputs_from(la, q, K, V, lens, H, d, dtype):
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    return W.Inputs(q=q.to(tdt).cuda().contiguous(), k=K.to(tdt).cuda().contiguous(),
                    v=V.to(tdt).cuda().contiguous(), ctx_lens=lens, H=H, d=d, dtype=dtype,
                    scale=1.0 / math.sqrt(d), seed=0)


@pytest.mark.parametrize("kind", KINDS)
def test_closed_forms(la, kind):
    g = torch.Generator().manual_seed(1)
    H, d = 2, 128
    lens = [1, 5000]
    N = sum(lens)
    q = torch.randn((2, H, d), generator=g)
    K = torch.randn((H * N, d), generator=g)
    # constant V: the output is that constant
    c = torch.randn(d, generator=g).to(torch.bfloat16).float()
    inp = _inputs_from(la, q, K, c.expand(H * N, d), lens, H, d, "bf16")
    O, m, l = run(la, inp, kind)
    assert np.max(np.abs(O - c.numpy())) <= 1e-4
    # one token: O = V_0 and l = 1 (request 0 has n = 1)
    V = torch.randn((H * N, d), generator=g)
    inp = _inputs_from(la, q, K, V, lens, H, d, "bf16")
    O, m, l = run(la, inp, kind)
    v0 = inp.v[:H].float().cpu().numpy()
    assert np.max(np.abs(O[0] - v0)) <= 1e-6 and np.all(l[0] == 1.0)
    # q = 0: m = 0, l = n, O = the mean of V
    inp = _inputs_from(la, torch.zeros_like(q), K, V, lens, H, d, "bf16")
    O, m, l = run(la, inp, kind)
    Vb = inp.v.float().cpu().numpy()
    mean = Vb[H:H + 5000].mean(axis=0)
    assert np.max(np.abs(O[1, 0] - mean)) <= 1e-4
    assert np.all(m == 0.0) and abs(l[1, 0] - 5000) <= 5000 * 1e-5
    # a dominant logit: O = that V row
    Kd = K.clone()
    j = 4321
    qn = q[1, 0].norm()
    Kd[H + j] = (100.0 * math.sqrt(d) / qn) * (q[1, 0] / qn)    # s_j = 100, others ~ N(0, 1)
    inp = _inputs_from(la, q, Kd, V, lens, H, d, "bf16")
    O, m, l = run(la, inp, kind)
    assert np.max(np.abs(O[1, 0] - inp.v[H + j].float().cpu().numpy())) <= 1e-4
    assert 1.0 <= float(l[1, 0]) <= 1.0 + 1e-4


def test_determinism(la):
    inp = W.make_custom([777, 31000, 1], H=6, d=128, dtype="bf16", seed=8, device="cuda")
    first = run(la, inp, "lean")
    for _ in range(20):
        again = run(la, inp, "lean")
        for a, b in zip(first, again):
            assert np.array_equal(a, b, equal_nan=True)


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "f16")])
def test_wide_merge(la, d, dtype):
    """Heads spread over many workgroups: a host with more than 16 peers
    merges on all four waves, each folding a quarter of the peers, then wave
    0 folds the waves' states in wave order. The result meets the oracle and
    is bitwise the same from launch to launch (the order is fixed)."""
    cap = la.la_max_grid(d, la.LA_BF16 if dtype == "bf16" else la.LA_F16)
    for lens, H, grid in (([200000], 1, 256), ([100000, 3], 2, cap), ([70000], 1, 19)):
        inp = W.make_custom(lens, H=H, d=d, dtype=dtype, seed=31, device="cuda")
        say(f"[wide merge] d={d} lens={lens} H={H} grid={grid}")
        first = run(la, inp, "lean", grid=grid)
        check(first, reference(inp), tag=f"wide/{lens}/{grid}")
        for _ in range(5):
            again = run(la, inp, "lean", grid=grid)
            for a, b in zip(first, again):
                assert np.array_equal(a, b, equal_nan=True)


def test_timeout_path_recovers(la):
    """A 1 us wait bound makes hosts give up waiting (forced from the host);
    the launch still ends, la_sync_check reports or not, and after the reset
    the next call is exact again."""
    inp = W.make_custom([30000, 30000], H=2, d=128, dtype="bf16", seed=2, device="cuda")
    try:
        la.la_set_wait_limit_us(1)
        for _ in range(3):
            out = torch.empty((2, 2, 128), dtype=torch.float32, device="cuda")
            la.la_decode_ex(inp.q, inp.k, inp.v, inp.ctx_lens, 2, 2, 128, inp.scale, out)
            try:
                la.la_sync_check()
            except la.LaError as e:
                assert e.status == 4
    finally:
        la.la_set_wait_limit_us(0)
    check(run(la, inp, "lean"), reference(inp), tag="after-timeout")


def _late_peer_case():
    """Tiles of 8192 tokens, grid 3. Request 0 has one token per head (one
    tile each), request 1 five full tiles per schedule unit. Workgroup 0's
    range starts with request 0's tiny tiles and ends with the first tiles of
    request 1's first unit, which it hosts; its first peer streams one full
    tile more than it before publishing (2 against 1 with one unit per
    request, 3 against 2 with two). The host so reaches its wait tens of
    microseconds early, and a 1 us bound always gives up."""
    return [1, 8192 * 5], dict(tile_tokens=8192, grid=3)


@pytest.mark.parametrize("H,Hk", [(2, 2), (4, 1)])
def test_timeout_stays_in_its_launch(la, H, Hk):
    """Hosts give up waiting in three launches (1 us bound, forced from the
    host); with the bound restored and no la_sync_check in between, the next
    launches are exact on every head: a give-up reaches no later launch.
    la_sync_check then reports the timeout once."""
    lens, opts = _late_peer_case()
    d = 128
    inp = W.make_custom(lens, H=H, d=d, dtype="bf16", seed=12, device="cuda", kv_heads=Hk)
    ref = reference_kv(inp)
    la.la_sync_check()
    out = torch.empty((inp.B, H, d), dtype=torch.float32, device="cuda")
    try:
        la.la_set_wait_limit_us(1)
        for _ in range(3):
            la.la_decode_ex(inp.q, inp.k, inp.v, inp.ctx_lens, inp.B, H, d, inp.scale, out,
                            kv_heads=Hk, **opts)
    finally:
        la.la_set_wait_limit_us(0)
    for i in range(2):
        out = torch.full((inp.B, H, d), float("nan"), dtype=torch.float32, device="cuda")
        m = torch.full((inp.B * H,), float("nan"), dtype=torch.float32, device="cuda")
        l = torch.full((inp.B * H,), float("nan"), dtype=torch.float32, device="cuda")
        la.la_decode_ex(inp.q, inp.k, inp.v, inp.ctx_lens, inp.B, H, d, inp.scale, out,
                        kv_heads=Hk, m_out=m, l_out=l, **opts)
        torch.cuda.synchronize()
        check((out.cpu().numpy(), m.view(inp.B, H).cpu().numpy(), l.view(inp.B, H).cpu().numpy()),
              ref, tag=f"after-timeout launch {i}")
    with pytest.raises(la.LaError) as e:
        la.la_sync_check()
    assert e.value.status == 4
    la.la_sync_check()      # reported once, then clear


# ------------------------------------------------------------------ full-size workloads

# the ragged batch also at two more seeded draws of its lengths
@pytest.mark.parametrize("name,seed", [("65k", 0), ("512k", 0), ("ragged", 0), ("ragged", 2),
                                       ("ragged", 3), ("many-heads", 0), ("512k-h4", 0)])
def test_full_size(la, name, seed):
    """Every kind on the full workload, every (request, head) against the
    oracle; the lean kernel's executed tile map against the schedule oracle."""
    say(f"[full {name} seed {seed}] generating")
    inp = W.make_inputs(name, seed=seed, device="cuda")
    w = inp.meta["workload"]
    say(f"[full {name}] lens={inp.ctx_lens[:4]}... all {inp.B * inp.H} heads checked")
    res = {}
    for kind in KINDS:
        res[kind] = run(la, inp, kind)
        say(f"[full {name}] {kind} done")
    ref = full_reference(name, seed, inp)
    say(f"[full {name}] oracle done")
    for kind in KINDS:
        err = check(res[kind], ref, tag=f"{name}/{kind}")
        say(f"[full {name}] {kind} max|dO|={err:.2e}")
    # the lean kernel executed the oracle's tile map
    L = la.la_default_tile(w.d)
    G_req = la.la_default_grid(w.d, la.LA_BF16 if w.dtype == "bf16" else la.LA_F16)
    own_ref, G = tile_owner_ref(inp.ctx_lens, inp.H, L, G_req)
    owner = torch.full((own_ref.size,), -1, dtype=torch.int32, device="cuda")
    run(la, inp, "lean", tile_owner=owner)
    assert np.array_equal(owner.cpu().numpy(), own_ref)
    del inp
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ edge cases

@pytest.mark.parametrize("kind", KINDS)
def test_all_single_token_requests(la, kind):
    lens = [1] * 37
    inp = W.make_custom(lens, H=5, d=64, dtype="f16", seed=31, device="cuda")
    check(run(la, inp, kind), reference(inp), tag=f"n=1/{kind}")


@pytest.mark.parametrize("kind", KINDS)
def test_many_small_requests(la, kind):
    """512 requests of 1..300 tokens: each lean workgroup holds many segments
    (whole heads between a peer segment and a host segment)."""
    rng = np.random.default_rng(4)
    lens = [int(x) for x in rng.integers(1, 301, size=512)]
    inp = W.make_custom(lens, H=2, d=128, dtype="bf16", seed=41, device="cuda")
    check(run(la, inp, kind), reference(inp), tag=f"many-small/{kind}")


@pytest.mark.parametrize("B", [255, 256, 257, 600, 1024, 1025])
def test_schedule_source_across_the_inline_limit(la, B):
    """Up to 256 requests the workgroups derive their segments from prefix
    sums in the kernel arguments, up to 1024 from the lengths copied to the
    device, above that they read the host's tables: on every side of both
    limits the tile map is the oracle's, and forcing the tables gives the
    same bits."""
    rng = np.random.default_rng(B)
    lens = [int(x) for x in rng.integers(1, 700, size=B)]
    H, d = 2, 64
    inp = W.make_custom(lens, H=H, d=d, dtype="f16", seed=B, device="cuda")
    L = la.la_default_tile(d)
    for grid in (0, 97):
        G_req = grid if grid else la.la_default_grid(d, la.LA_F16)
        own_ref, _ = tile_owner_ref(lens, H, L, G_req)
        say(f"[inline limit B={B} grid={grid}]")
        owner = torch.full((own_ref.size,), -1, dtype=torch.int32, device="cuda")
        a = run(la, inp, "lean", grid=grid, tile_owner=owner)
        assert np.array_equal(owner.cpu().numpy(), own_ref)
        b = run(la, inp, "lean", grid=grid, host_tables=True)
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)
    check(a, reference(inp), tag=f"B={B}")


@pytest.mark.parametrize("tile", [(1 << 20), (1 << 31) - 1])
@pytest.mark.parametrize("kind,opts", [("lean", {}), ("lean", {"host_tables": True}),
                                       ("pull", {"grid": 3}), ("chunks", {}),
                                       ("fixed_split", {"num_splits": 4})])
def test_tile_larger_than_every_context(la, tile, kind, opts):
    """A LeanTile longer than any context (up to the largest int): one tile
    per head, no overflow in the tile counts or token offsets."""
    lens = [700, 1, 5000]
    inp = W.make_custom(lens, H=3, d=64, dtype="f16", seed=44, device="cuda")
    say(f"[huge tile {tile} {kind} {opts}]")
    check(run(la, inp, kind, tile_tokens=tile, **opts), reference(inp), tag=f"L={tile}/{kind}")


def test_grid_larger_than_work(la):
    """Fewer tile iterations than the requested grid: G is cut to I."""
    lens = [3, 200]
    inp = W.make_custom(lens, H=2, d=128, dtype="bf16", seed=43, device="cuda")
    grid = la.la_max_grid(128, la.LA_BF16)     # the largest grid a launch may ask for
    own_ref, G = tile_owner_ref(lens, 2, 16, grid)
    assert G == own_ref.size < grid
    owner = torch.full((own_ref.size,), -1, dtype=torch.int32, device="cuda")
    check(run(la, inp, "lean", grid=grid, tile_tokens=16, tile_owner=owner), reference(inp),
          tag="G>I")
    assert np.array_equal(owner.cpu().numpy(), own_ref)


def test_largest_head(la):
    """One head at the 4 GiB limit of a head's block (n = 2^24 - 1 at d = 128):
    the last rows sit right below the 32-bit offset boundary."""
    n = (1 << 24) - 1
    say(f"[largest head] n={n}")
    inp = W.make_custom([n], H=1, d=128, dtype="bf16", seed=47, device="cuda")
    got = {k: run(la, inp, k) for k in ("lean", "fixed_split")}
    ref = sampled_reference(inp, [(0, 0)])
    for k, g in got.items():
        check(g, ref, heads=[(0, 0)], tag=f"largest/{k}")
    del inp
    torch.cuda.empty_cache()


def test_rejects_without_launch(la):
    inp = W.make_custom([4, 4], H=1, d=128, dtype="bf16", seed=1, device="cuda")
    out = torch.empty((2, 1, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(la.LaError) as e:
        la.la_decode_ex(inp.q, inp.k, inp.v, [4, 0], 2, 1, 128, 0.1, out)
    assert e.value.status == 1
    cap = la.la_max_grid(128, la.LA_BF16)
    with pytest.raises(la.LaError) as e:
        la.la_decode_ex(inp.q, inp.k, inp.v, [4, 4], 2, 1, 128, 0.1, out, grid=cap + 1)
    assert e.value.status == 1
    la.la_sync_check()


@pytest.mark.parametrize("kind,blocks", [("lean", None), ("fixed_split", 4), ("per_head", None)])
def test_timestamps(la, kind, blocks):
    lens = [20000, 3000]
    H, d = 4, 128
    inp = W.make_custom(lens, H=H, d=d, dtype="bf16", seed=53, device="cuda")
    opts = {}
    if kind == "lean":
        _, n, _ = la.la_schedule_dims(lens, H, la.la_default_tile(d), la.la_default_grid(d, la.LA_BF16))
    elif kind == "fixed_split":
        n = len(lens) * H * blocks
        opts["num_splits"] = blocks
    else:
        n = len(lens) * H
    ts = torch.zeros(n * 4, dtype=torch.int64, device="cuda")
    got = run(la, inp, kind, cta_timestamps=ts, **opts)
    check(got, reference(inp), tag=f"timestamps/{kind}")
    a = ts.view(n, 4).cpu().numpy()
    assert np.all(a[:, 0] > 0) and np.all(a[:, 1] >= a[:, 0])
    span_us = (a[:, 1].max() - a[:, 0].min()) / 100.0
    assert 0 < span_us < 1e6
    if kind != "lean":
        assert np.all(a[:, 3] == 0)
        return
    # the fourth word: a split unit's host, when its wait for the peers began
    # and ended (ticks after entry); 0 for the other workgroups
    s = oracle.lean_schedule(lens, H, la.la_default_tile(d), la.la_default_grid(d, la.LA_BF16))
    hosts = {c for (c, u, t0, t1, h, f) in s["seg"] if h and not f}
    assert hosts
    w = a[:, 3].astype(np.uint64)
    begin, end = (w & np.uint64(0xFFFFFFFF)).astype(np.int64), (w >> np.uint64(32)).astype(np.int64)
    for c in range(n):
        if c in hosts:
            assert 0 < begin[c] <= end[c] <= a[c, 1] - a[c, 0], (c, begin[c], end[c])
        else:
            assert a[c, 3] == 0, c


def test_stream_capture_is_refused(la):
    """A stream being captured into a graph before any call has sized its
    workspace is refused before anything is enqueued."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")
    inp = W.make_custom([300, 40], H=2, d=64, dtype="f16", seed=61, device="cuda")
    out = torch.empty((2, 2, 64), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    hip.hipStreamBeginCapture.argtypes = [ctypes.c_void_p, ctypes.c_int]
    hip.hipStreamEndCapture.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
    hip.hipGraphDestroy.argtypes = [ctypes.c_void_p]
    assert hip.hipStreamBeginCapture(ctypes.c_void_p(s.cuda_stream), 2) == 0   # relaxed mode
    try:
        with pytest.raises(la.LaError) as e:
            la.la_decode_ex(inp.q, inp.k, inp.v, inp.ctx_lens, 2, 2, 64, inp.scale, out,
                            stream=s.cuda_stream)
    finally:
        graph = ctypes.c_void_p()
        assert hip.hipStreamEndCapture(ctypes.c_void_p(s.cuda_stream), ctypes.byref(graph)) == 0
        if graph.value:
            hip.hipGraphDestroy(graph)
    assert e.value.status == 2 and "capture" in str(e.value)
    # the stream works normally afterwards
    la.la_decode_ex(inp.q, inp.k, inp.v, inp.ctx_lens, 2, 2, 64, inp.scale, out,
                    stream=s.cuda_stream)
    s.synchronize()
    O = out.cpu().numpy()
    Or = reference(inp)[0]
    assert float(np.max(np.abs(O - Or))) <= 1e-3
