"""GPU parity for the dynamic-pull kinds: fixed chunks of the lean tile
sequence, pulled from an atomic counter by a persistent grid (pull) or one per
workgroup (chunks), heads spread over chunks merged by the last piece's
workgroup. Same bar as the other kernels against the fp64 oracle; outputs are
bitwise independent of the grid and of which workgroup took which chunk."""
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


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def la():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_phase_attention_amd as la
    la.lib()
    return la


def run(la, inp, kind, owner=None, **opts):
    B, H, d = inp.B, inp.H, inp.d
    out = torch.full((B, H, d), float("nan"), dtype=torch.float32, device="cuda")
    m = torch.full((B * H,), float("nan"), dtype=torch.float32, device="cuda")
    l = torch.full((B * H,), float("nan"), dtype=torch.float32, device="cuda")
    la.la_decode_ex(inp.q, inp.k, inp.v, inp.ctx_lens, B, H, d, inp.scale, out, kind=kind,
                    m_out=m, l_out=l, tile_owner=owner, **opts)
    la.la_sync_check()
    return out.cpu().numpy(), m.view(B, H).cpu().numpy(), l.view(B, H).cpu().numpy()


def reference(inp, heads=None):
    return oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), inp.ctx_lens,
                              inp.scale, inp.dtype, heads=heads, workers=16)


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


def tiles(lens, H, L):
    return H * sum((n + L - 1) // L for n in lens)


def check_owner(owner, I, C, kind, grid=None):
    """Every tile was processed, a chunk by one workgroup; chunks: chunk k by
    workgroup k; pull: only workgroups of the grid."""
    own = owner.cpu().numpy()
    assert own.shape == (I,) and (own >= 0).all()
    nch = (I + C - 1) // C
    per_chunk = np.pad(own, (0, nch * C - I), constant_values=-1).reshape(nch, C)
    for k in range(nch):
        vals = set(per_chunk[k][per_chunk[k] >= 0].tolist())
        assert len(vals) == 1, (k, vals)
        if kind == "chunks":
            assert vals == {k}
        else:
            assert next(iter(vals)) < grid


CASES = [([3000, 17, 60000, 129, 4096, 2176], 4, 128, "bf16"),
         ([1, 700, 256, 2049], 8, 64, "f16"),
         ([20000], 32, 128, "f16")]


@pytest.mark.parametrize("lens,H,d,dtype", CASES)
@pytest.mark.parametrize("C", [1, 3, 16, 200])
def test_chunks_parity_and_tile_map(la, lens, H, d, dtype, C):
    say(f"[chunks] lens={lens} H={H} d={d} {dtype} C={C}")
    inp = W.make_custom(lens, H, d, dtype, seed=C + H, device="cuda")
    ref = reference(inp)
    L = la.la_default_tile(d)
    I = tiles(lens, H, L)
    owner = torch.full((I,), -1, dtype=torch.int32, device="cuda")
    check(run(la, inp, "chunks", owner, chunk_tiles=C), ref, tag=f"chunks C={C}")
    check_owner(owner, I, C, "chunks")


@pytest.mark.parametrize("lens,H,d,dtype", CASES)
@pytest.mark.parametrize("grid,C", [(1, 5), (7, 1), (64, 4), (256, 0), (3000, 2)])
def test_pull_parity_and_tile_map(la, lens, H, d, dtype, grid, C):
    say(f"[pull] lens={lens} H={H} d={d} {dtype} grid={grid} C={C}")
    inp = W.make_custom(lens, H, d, dtype, seed=grid + C, device="cuda")
    ref = reference(inp)
    L = la.la_default_tile(d)
    I = tiles(lens, H, L)
    owner = torch.full((I,), -1, dtype=torch.int32, device="cuda")
    check(run(la, inp, "pull", owner, grid=grid, chunk_tiles=C), ref, tag=f"pull grid={grid}")
    Ceff = C if C > 0 else max(min(32, -(-I // grid)), -(-I // (8 * grid)))
    check_owner(owner, I, Ceff, "pull", grid)


def test_bitwise_independent_of_grid_and_assignment(la):
    inp = W.make_custom([50000, 3000, 90000], 16, 128, "bf16", seed=5, device="cuda")
    base = run(la, inp, "chunks", chunk_tiles=9)
    for grid in (1, 13, 256, 1024, 5000):
        for _ in range(2):
            got = run(la, inp, "pull", grid=grid, chunk_tiles=9)
            for x, y in zip(base, got):
                np.testing.assert_array_equal(x, y)


def test_back_to_back_reuses_counters(la):
    """The counters are re-armed by each launch: many launches of different
    shapes and grids in a row, no synchronisation between them."""
    a = W.make_custom([5000, 300, 12000], 8, 128, "bf16", seed=6, device="cuda")
    b = W.make_custom([700] * 9, 4, 64, "f16", seed=7, device="cuda")
    ra, rb = reference(a), reference(b)
    outs = []
    for i in range(24):
        inp = a if i % 2 == 0 else b
        out = torch.full((inp.B, inp.H, inp.d), float("nan"), dtype=torch.float32, device="cuda")
        kind = "pull" if i % 3 else "chunks"
        la.la_decode_ex(inp.q, inp.k, inp.v, inp.ctx_lens, inp.B, inp.H, inp.d, inp.scale, out,
                        kind=kind, grid=(0 if kind == "chunks" else 1 + 37 * i), chunk_tiles=1 + i % 5)
        outs.append((i, out))
    la.la_sync_check()
    for i, out in outs:
        ref = ra if i % 2 == 0 else rb
        err = float(np.max(np.abs(out.cpu().numpy() - ref[0])))
        assert err <= O_TOL, (i, err)


@pytest.mark.parametrize("H,Hk,Nq,d,dtype", [(8, 2, 1, 64, "f16"), (32, 8, 1, 128, "bf16"),
                                              (4, 4, 4, 128, "bf16"), (16, 2, 3, 64, "f16")])
@pytest.mark.parametrize("kind,grid,C", [("pull", 0, 0), ("pull", 5, 1), ("pull", 700, 3),
                                         ("chunks", 0, 2), ("chunks", 0, 40)])
def test_grouped_and_several_tokens(la, H, Hk, Nq, d, dtype, kind, grid, C):
    """The grouped MFMA kernel pulled the same way: units (K/V head, block of
    16 query columns) instead of heads."""
    L = la.la_default_tile(d)
    lens = [Nq, 3 * L + 1, 5000, 700]
    say(f"[pull grouped] H={H} Hk={Hk} Nq={Nq} d={d} {kind} grid={grid} C={C}")
    inp = W.make_custom(lens, H, d, dtype, seed=H + Hk + Nq + C, device="cuda", kv_heads=Hk,
                        q_tokens=Nq)
    ref = oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), lens,
                             inp.scale, dtype, workers=16, kv_heads=Hk)
    shape = tuple(inp.q.shape)
    out = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    rows = int(np.prod(shape[:-1]))
    m = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    l = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    U = Hk * ((H // Hk * Nq + 15) // 16)
    I = U * sum((n + L - 1) // L for n in lens)
    owner = torch.full((I,), -1, dtype=torch.int32, device="cuda")
    la.la_decode_ex(inp.q, inp.k, inp.v, lens, len(lens), H, d, inp.scale, out, kind=kind,
                    grid=grid, chunk_tiles=C, m_out=m, l_out=l, tile_owner=owner, kv_heads=Hk,
                    q_tokens=Nq)
    la.la_sync_check()
    check((out.cpu().numpy(), m.cpu().numpy().reshape(ref[1].shape),
           l.cpu().numpy().reshape(ref[2].shape)), ref, tag=f"grouped {kind}")
    G = grid if grid > 0 else la.la_default_grid(d, la.LA_BF16 if dtype == "bf16" else la.LA_F16)
    # the default chunk for grouped units: four per workgroup of the grid
    Ceff = C if C > 0 else max(min(32, -(-I // G)), -(-I // (4 * G)))
    check_owner(owner, I, Ceff, kind, grid if kind == "pull" and grid > 0 else 1 << 30)


@pytest.mark.parametrize("name", ["512k", "ragged", "gqa8-ragged", "spec4-ragged"])
def test_full_size(la, name):
    say(f"[pull full {name}]")
    inp = W.make_inputs(name, seed=0, device="cuda")
    Nq = inp.Nq
    ref = full_reference(name, 0, inp)      # every query row
    shape = tuple(inp.q.shape)
    rows = int(np.prod(shape[:-1]))
    for kind in ("pull", "chunks"):
        out = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
        m = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
        l = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
        la.la_decode_ex(inp.q, inp.k, inp.v, inp.ctx_lens, inp.B, inp.H, inp.d, inp.scale, out,
                        kind=kind, m_out=m, l_out=l, kv_heads=inp.Hk, q_tokens=Nq)
        la.la_sync_check()
        got = (out.cpu().numpy(), m.cpu().numpy().reshape(ref[1].shape),
               l.cpu().numpy().reshape(ref[2].shape))
        err = check(got, ref, tag=f"{name}/{kind}")
        say(f"[pull full {name}] {kind} max|dO|={err:.2e}")
    del inp
    torch.cuda.empty_cache()
