"""GPU parity for grouped-query heads (GQA/MQA): the MFMA kernels through the
C ABI against the fp64 oracle, same bar as the single-head kernels (max |dO|
<= 1e-3, l within 1e-5 relative after rescaling to the oracle's max, m within
1e-5), and the executed tile-to-workgroup map bit-exact."""
from __future__ import annotations

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
KINDS = ["lean", "fixed_split", "per_head"]


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
    out = torch.full((B, H, d), float("nan"), dtype=torch.float32, device="cuda")
    m = torch.full((B * H,), float("nan"), dtype=torch.float32, device="cuda")
    l = torch.full((B * H,), float("nan"), dtype=torch.float32, device="cuda")
    la.la_decode_ex(inp.q, inp.k, inp.v, inp.ctx_lens, B, H, d, inp.scale, out, kind=kind,
                    m_out=m, l_out=l, kv_heads=inp.Hk, **opts)
    la.la_sync_check()
    return out.cpu().numpy(), m.view(B, H).cpu().numpy(), l.view(B, H).cpu().numpy()


def reference(inp, heads=None):
    return oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), inp.ctx_lens,
                              inp.scale, inp.dtype, heads=heads, workers=16, kv_heads=inp.Hk)


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


@pytest.mark.parametrize("H,Hk", [(6, 3), (12, 4), (8, 2), (16, 2), (16, 1), (32, 1)])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64), ("f16", 128), ("bf16", 64)])
def test_groups_ragged(la, H, Hk, dtype, d):
    lens = [1, 7, 129, 1000, 4097, 300]
    inp = W.make_custom(lens, H=H, d=d, dtype=dtype, seed=61, device="cuda", kv_heads=Hk)
    ref = reference(inp)
    for kind in KINDS:
        say(f"[gqa H={H} Hk={Hk} {dtype} d={d} {kind}]")
        check(run(la, inp, kind), ref, tag=f"H={H}/Hk={Hk}/{dtype}/{d}/{kind}")


@pytest.mark.parametrize("host_tables", [False, True])
@pytest.mark.parametrize("grid", [1, 3, 37, 0])
@pytest.mark.parametrize("tile", [0, 32, 200])
def test_schedule_invariance_and_tile_map(la, grid, tile, host_tables):
    lens = [33, 1, 700, 2048, 5]
    H, Hk, d = 24, 2, 128            # g = 12: one query block per K/V head
    inp = W.make_custom(lens, H=H, d=d, dtype="bf16", seed=62, device="cuda", kv_heads=Hk)
    L = tile if tile else la.la_default_tile(d)
    units = Hk * 1
    G_req = grid if grid else la.la_default_grid(d, la.LA_BF16)
    s = oracle.lean_schedule(lens, units, L, G_req)
    own = np.empty(s["I"], np.int32)
    for (c, u, t0, t1, _h, _f) in s["seg"]:
        own[s["S"][u] + t0:s["S"][u] + t1] = c
    owner = torch.full((own.size,), -1, dtype=torch.int32, device="cuda")
    got = run(la, inp, "lean", grid=grid, tile_tokens=tile, tile_owner=owner,
              host_tables=host_tables)
    check(got, reference(inp), tag=f"grid={grid} tile={tile}")
    assert np.array_equal(owner.cpu().numpy(), own)


def test_two_query_blocks_tile_map(la):
    """g = 20 > 16: every K/V head is two schedule units (16 + 4 query heads)."""
    lens = [500, 3000]
    H, Hk, d = 40, 2, 64
    inp = W.make_custom(lens, H=H, d=d, dtype="f16", seed=63, device="cuda", kv_heads=Hk)
    L = la.la_default_tile(d)
    s = oracle.lean_schedule(lens, Hk * 2, L, 11)
    own = np.empty(s["I"], np.int32)
    for (c, u, t0, t1, _h, _f) in s["seg"]:
        own[s["S"][u] + t0:s["S"][u] + t1] = c
    owner = torch.full((own.size,), -1, dtype=torch.int32, device="cuda")
    check(run(la, inp, "lean", grid=11, tile_owner=owner), reference(inp), tag="g=20")
    assert np.array_equal(owner.cpu().numpy(), own)


def test_adversarial_scores(la):
    for dtype in ("f16", "bf16"):
        inp = W.make_custom([3000, 20000], H=16, d=128, dtype=dtype, seed=64, device="cuda",
                            q_std=6.0, kv_heads=2)
        check(run(la, inp, "lean", grid=29), reference(inp), tag=f"adversarial/{dtype}")


@pytest.mark.parametrize("host_tables", [False, True])
def test_host_wait_timestamps(la, host_tables):
    """Per-workgroup timestamps of the grouped lean kernel: every workgroup
    that hosts a split unit records when its wait for the peers began and
    ended, within its own entry and exit; the others record 0."""
    lens = [9000, 40, 3000]
    H, Hk, d = 16, 4, 64
    inp = W.make_custom(lens, H=H, d=d, dtype="f16", seed=64, device="cuda", kv_heads=Hk)
    G_req = 37
    s = oracle.lean_schedule(lens, Hk, la.la_default_tile(d), G_req)
    G = s["G"]
    hosts = {c for (c, u, t0, t1, h, f) in s["seg"] if h and not f}
    assert hosts
    ts = torch.zeros(G * 4, dtype=torch.int64, device="cuda")
    check(run(la, inp, "lean", grid=G_req, cta_timestamps=ts, host_tables=host_tables),
          reference(inp), tag="timestamps")
    a = ts.view(G, 4).cpu().numpy()
    w = a[:, 3].astype(np.uint64)
    begin = (w & np.uint64(0xFFFFFFFF)).astype(np.int64)
    end = (w >> np.uint64(32)).astype(np.int64)
    for c in range(G):
        if c in hosts:
            assert 0 < begin[c] <= end[c] <= a[c, 1] - a[c, 0], (c, begin[c], end[c])
        else:
            assert a[c, 3] == 0, c


def test_determinism(la):
    inp = W.make_custom([777, 31000, 1], H=32, d=128, dtype="bf16", seed=65, device="cuda",
                        kv_heads=8)
    first = run(la, inp)
    for _ in range(10):
        again = run(la, inp)
        for a, b in zip(first, again):
            assert np.array_equal(a, b, equal_nan=True)


def test_random_grids_stress(la):
    lens = [300000, 3, 50000]
    inp = W.make_custom(lens, H=16, d=128, dtype="bf16", seed=66, device="cuda", kv_heads=2)
    ref, _, _ = reference(inp)
    cap = la.la_default_grid(128, la.LA_BF16)
    rng = np.random.default_rng(9)
    out = torch.empty((3, 16, 128), dtype=torch.float32, device="cuda")
    for i, g in enumerate([cap, 1, 2] + [int(x) for x in rng.integers(1, cap + 1, 60)]):
        out.fill_(float("nan"))
        la.la_decode_ex(inp.q, inp.k, inp.v, lens, 3, 16, 128, inp.scale, out, grid=g,
                        kv_heads=2)
        la.la_sync_check()
        err = float(np.max(np.abs(out.cpu().numpy() - ref)))
        assert err <= O_TOL, (i, g, err)


@pytest.mark.parametrize("name,seed", [("gqa-512k", 0), ("gqa8-ragged", 0), ("gqa8-ragged", 3),
                                       ("mqa-32k", 0)])
def test_full_size(la, name, seed):
    """Every kind on the full workload (the grouped ragged batch also at a
    second draw of its lengths), every (request, query head) against the
    oracle."""
    say(f"[gqa full {name} seed {seed}]")
    inp = W.make_inputs(name, seed=seed, device="cuda")
    res = {k: run(la, inp, k) for k in KINDS}
    ref = full_reference(name, seed, inp)
    for k in KINDS:
        err = check(res[k], ref, tag=f"{name}/{k}")
        say(f"[gqa full {name}] {k} max|dO|={err:.2e}")
    del inp
    torch.cuda.empty_cache()


def _inputs(q, K, V, lens, H, Hk, d, dtype):
    import math
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    return W.Inputs(q=q.to(tdt).cuda().contiguous(), k=K.to(tdt).cuda().contiguous(),
                    v=V.to(tdt).cuda().contiguous(), ctx_lens=lens, H=H, d=d, dtype=dtype,
                    scale=1.0 / math.sqrt(d), seed=0, meta={"kv_heads": Hk})


@pytest.mark.parametrize("kind,opts", [("lean", {}), ("lean", {"grid": 64}), ("lean", {"grid": 5}),
                                       ("fixed_split", {"num_splits": 7}), ("per_head", {}),
                                       ("pull", {"grid": 9})])
@pytest.mark.parametrize("H,Hk,d", [(4, 1, 128), (8, 4, 128), (16, 1, 64)])
def test_closed_forms(la, kind, opts, H, Hk, d):
    """Results the definition fixes exactly, on the grouped kernels with heads
    split over many workgroups: constant V gives that constant; a one-token
    request gives its V row and l = 1 for every query head of the group; q = 0
    gives m = 0, l = n and the mean of V; one dominant logit of one query head
    gives that V row for that head only."""
    import math
    g = torch.Generator().manual_seed(3)
    lens = [1, 5000]
    N = sum(lens)
    q = torch.randn((2, H, d), generator=g)
    K = torch.randn((Hk * N, d), generator=g)
    c = torch.randn(d, generator=g).to(torch.bfloat16).float()
    say(f"[closed forms] {kind} {opts} H={H} Hk={Hk} d={d}")
    inp = _inputs(q, K, c.expand(Hk * N, d), lens, H, Hk, d, "bf16")
    O, m, l = run(la, inp, kind, **opts)
    assert np.max(np.abs(O - c.numpy())) <= 1e-4
    V = torch.randn((Hk * N, d), generator=g)
    inp = _inputs(q, K, V, lens, H, Hk, d, "bf16")
    O, m, l = run(la, inp, kind, **opts)
    grp = H // Hk
    v = inp.v.float().cpu().numpy()
    for h in range(H):
        assert np.max(np.abs(O[0, h] - v[h // grp])) <= 1e-6 and l[0, h] == 1.0
    inp = _inputs(torch.zeros_like(q), K, V, lens, H, Hk, d, "bf16")
    O, m, l = run(la, inp, kind, **opts)
    v = inp.v.float().cpu().numpy()
    for h in range(H):
        kv = h // grp
        rows = v[Hk * 1 + kv * 5000:Hk * 1 + (kv + 1) * 5000]
        assert np.max(np.abs(O[1, h] - rows.mean(axis=0))) <= 1e-4
        assert abs(l[1, h] - 5000) <= 5000 * 1e-5
    assert np.all(m == 0.0)
    Kd = K.clone()
    h0, j = H - 1, 4321
    kv0 = h0 // grp
    qn = q[1, h0].norm()
    row = Hk * 1 + kv0 * 5000 + j
    Kd[row] = (100.0 * math.sqrt(d) / qn) * (q[1, h0] / qn)     # s_j = 100 for head h0
    inp = _inputs(q, Kd, V, lens, H, Hk, d, "bf16")
    O, m, l = run(la, inp, kind, **opts)
    assert np.max(np.abs(O[1, h0] - inp.v[row].float().cpu().numpy())) <= 1e-4
    assert 1.0 <= float(l[1, h0]) <= 1.0 + 1e-4
    ref = reference(inp)
    check((O, m, l), ref, tag=f"dominant/{kind}")


@pytest.mark.parametrize("B", [300, 1024, 1025])
def test_copied_lengths_and_tables_agree(la, B):
    """Grouped heads with more requests than the kernel arguments hold: up to
    1024 the launch derives the partition from lengths copied to the device,
    above that from the host's tables. The tile map is the oracle's and
    forcing the tables gives the same bits."""
    rng = np.random.default_rng(B + 7)
    lens = [int(x) for x in rng.integers(1, 400, size=B)]
    H, Hk, d = 8, 2, 64
    inp = W.make_custom(lens, H=H, d=d, dtype="f16", seed=B, device="cuda", kv_heads=Hk)
    L = la.la_default_tile(d)
    for grid in (0, 61):
        G_req = grid if grid else la.la_default_grid(d, la.LA_F16)
        s = oracle.lean_schedule(lens, Hk, L, G_req)
        own = np.empty(s["I"], np.int32)
        for (c, u, t0, t1, _h, _f) in s["seg"]:
            own[s["S"][u] + t0:s["S"][u] + t1] = c
        say(f"[copied lengths B={B} grid={grid}]")
        owner = torch.full((own.size,), -1, dtype=torch.int32, device="cuda")
        a = run(la, inp, "lean", grid=grid, tile_owner=owner)
        assert np.array_equal(owner.cpu().numpy(), own)
        b = run(la, inp, "lean", grid=grid, host_tables=True)
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)
    check(a, reference(inp), tag=f"B={B}")


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "f16")])
def test_step_grid_phase(la, d, dtype):
    """The grouped lean kernel starts each segment's step grid at the 4 KiB
    boundary of the K rows at or before the segment start, masking the keys of
    the first step that precede it. Caches placed at every row offset within
    4 KiB, with tiles and grids that start segments at many rows, must give the
    oracle's result: a key counted twice or dropped at a segment start shows in
    l and O."""
    lens = [3, 130, 5000, 77, 2100]
    H, Hk = 8, 2
    inp = W.make_custom(lens, H=H, d=d, dtype=dtype, seed=88, device="cuda", kv_heads=Hk)
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
                        scale=inp.scale, seed=88, meta={"kv_heads": Hk})
        for opts in ({"tile_tokens": 48, "grid": 37}, {"tile_tokens": 32, "grid": 5},
                     {"grid": 3}, {}):
            say(f"[gqa phase d={d} offset={r} rows {opts}]")
            check(run(la, view, "lean", **opts), ref, tag=f"d={d}/offset={r}/{opts}")
